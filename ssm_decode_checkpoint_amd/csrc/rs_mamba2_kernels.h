// Mamba-2 decode kernels for gfx950: conventional read-modify-write step,
// ReplaySSM non-flush and flush steps, speculative append / commit (ReplaySSM
// and the snapshot baseline), and the NVFP4 read-copy quantizer.
//
// Per sequence b and head h (group g = h / heads_per_group), the layer is
//   a = exp(dt*A);  H = a*H + dt*x B^T;  y = H C + D*x
// and with checkpoint H0 and buffer entries 1..j (entry j the current token)
//   y_j = l_j (H0 C_j) + sum_i w_{j,i} dt_i (B_i.C_j) x_i + D x_j
//   fold: H = l_m H0 + sum_i (w_{m,i} dt_i x_i) B_i^T
// with l_j = prod_{l<=j} a_l and w_{j,i} = prod_{i<l<=j} a_l (sitech.ge
// ReplaySSM page, "How ReplaySSM works": outputs from checkpoint + buffer on
// non-flush steps, one checkpoint write per window on the flush step).
//
// Work decomposition: one 256-thread workgroup per (sequence, head) state
// matrix, stored transposed as [dstate][headdim] so that y = H C is a sum over
// rows that each thread accumulates in registers. The buffer records the
// workgroup needs (<= 16 x, B, dt and the current C) are staged in LDS while
// the state loads are in flight. Decay weights are direct products of the
// per-entry factors exp(dt*A).
#pragma once

#include "rs_device.h"
#include "rs_tile.h"
#include "rs_mtile.h"
#include "rs_internal.h"

namespace rs {

// ----------------------------------------------------------------------------
// staging of buffer records into LDS
// ----------------------------------------------------------------------------
// LDS of one Mamba-2 workgroup: NE buffer entries, Q outputs, and (XT) the
// fold coefficients. Sized per kernel so residency is not limited by LDS.
template <int NR, int NC, int NE, int Q, bool XT>
struct alignas(16) M2Smem {
  float B[NE][NR];
  float X[NE][NC];
  float Cw[Q][NR];        // C vectors the outputs are read with (current token, or drafts)
  float dt[NE];
  float a[NE];            // exp(dt*A)
  float w[Q][NE];         // per-output weights  w_{j,i} dt_i (B_i . C_j)
  float L[Q];             // l_j per output
  float red[4 * Q * NC];  // reduction scratch
  float out[Q * NC];      // matvec results
  alignas(16) float xt[XT ? NE : 1][NC];  // fold coefficients w_{m,i} dt_i x_i
  float s4[4];
};

// For outputs q = 0..nq-1 reading entries 0..J_q-1 (J_q = j0 + q):
//   L[q] = prod_{l<J_q} a_l;  w[q][e] = prod_{e<l<J_q} a_l * dt_e * (B_e . C_q)
// Dots use groups of 16 lanes (one per (q, e) pair per round).
template <typename SM>
__device__ __forceinline__ void output_weights(SM& s, int j0, int nq) {
  const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
  constexpr int NR = sizeof(s.B[0]) / sizeof(float);
  // valid pairs only: output q has J_q = j0 + q of them, q-major
  const int npairs = nq * j0 + nq * (nq - 1) / 2;
  for (int pair = grp; pair < npairs; pair += kThreads / 16) {
    int q = 0, e = pair;
    while (e >= j0 + q) {                        // uniform over the group
      e -= j0 + q;
      ++q;
    }
    const int J = j0 + q;
    float part = lds_dot16<NR>(&s.B[e][0], &s.Cw[q][0], ln);
    part = group_sum16(part);
    if (ln == 0) {
      float w = 1.0f;
      for (int l = e + 1; l < J; ++l) w *= s.a[l];
      s.w[q][e] = w * s.dt[e] * part;
    }
  }
  if (static_cast<int>(threadIdx.x) < nq) {
    const int J = j0 + threadIdx.x;
    float L = 1.0f;
    for (int l = 0; l < J; ++l) L *= s.a[l];
    s.L[threadIdx.x] = L;
  }
}

// ----------------------------------------------------------------------------
// conventional step (baseline): read + write the full state
// ----------------------------------------------------------------------------
template <typename TIN, int NR, int NC>
__global__ __launch_bounds__(kThreads) void m2_conv_kernel(M2Args a) {
  constexpr int E = 4;
  __shared__ M2Smem<NR, NC, 1, 1, false> s;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads, h = tile - b * a.nheads, g = h / a.hpg;
  static_assert(NR <= kThreads && NC <= kThreads, "one input element per thread");
  // the token's inputs into registers first, then the state (returns come back
  // in issue order), then the inputs to LDS while the state streams in
  const TIN* inB = static_cast<const TIN*>(a.B) + (static_cast<size_t>(b) * a.ngroups + g) * NR;
  const TIN* inC = static_cast<const TIN*>(a.C) + (static_cast<size_t>(b) * a.ngroups + g) * NR;
  const TIN* inX = static_cast<const TIN*>(a.x) + static_cast<size_t>(tile) * NC;
  const int ti = static_cast<int>(threadIdx.x);
  const int ir = ti < NR ? ti : 0, ic = ti < NC ? ti : 0;
  const float bv = to_f(inB[ir]), cv = to_f(inC[ir]), xv = to_f(inX[ic]);
  const float dt = to_f(static_cast<const TIN*>(a.dt)[tile]);
  const float Ah = a.A[h];
  RawTile<FMT_F32, E, NR, NC> raw;
  raw.issue(a.ck, tile);
  if (ti < NR) {
    s.B[0][ti] = bv;
    s.Cw[0][ti] = cv;
  }
  if (ti < NC) s.X[0][ti] = xv;
  __syncthreads();
  const float decay = expf(dt * Ah);
  RegTile<E, NR, NC> H;
  raw.decode(H);
  const int c0 = RegTile<E, NR, NC>::col0();
  float dtx[E];
#pragma unroll
  for (int i = 0; i < E; ++i) dtx[i] = dt * s.X[0][c0 + i];
#pragma unroll
  for (int k = 0; k < RegTile<E, NR, NC>::P; ++k) {
    const int row = RegTile<E, NR, NC>::row(k);
    if (row < NR) {
      const float br = s.B[0][row];
#pragma unroll
      for (int i = 0; i < E; ++i) H.v[k][i] = decay * H.v[k][i] + dtx[i] * br;
    }
  }
  tile_store<FMT_F32>(a.ck, tile, H, s.s4);
  tile_matvec<1>(H, &s.Cw[0][0], NR, s.red, s.out);
  for (int p = threadIdx.x; p < NC; p += kThreads)
    a.y[static_cast<size_t>(tile) * NC + p] = s.out[p] + a.D[h] * s.X[0][p];
}

// ----------------------------------------------------------------------------
// non-flush step: y from checkpoint (or read copy) + buffer; append; no state write
// ----------------------------------------------------------------------------
// Vector loads return in issue order. The buffer records this workgroup needs
// (<= 16 B and x rows, dt, the current C) are therefore loaded into registers
// first, the 32 KiB state tile right after them, and only then are the records
// moved to LDS: the state-independent work (decays, dots B_i . C_j, weights,
// the buffer part of y) runs while the tile streams in, and the tail after
// its arrival is one reduction and the y store.
template <int NR, int NC>
struct alignas(16) M2NfSmem {
  float B[kRing][NR];
  float X[kRing][NC];
  float C[NR];
  float dt[kRing];
  float a[kRing];            // prod_{i<l<j} exp(dt_l A): the decay from entry i to the current one
  float w[kRing];            // w_{j,i} dt_i (B_i . C_j)
  float L;
  float red[4 * NC];
  float out[NC];
};

template <typename TIN, int RDF, int NR, int NC>
__device__ __forceinline__ void m2_nonflush_body(const M2Args& a, M2NfSmem<NR, NC>& s) {
  constexpr int E = (RDF == FMT_F32) ? 4 : 8;
  constexpr int V = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NR % V == 0 && NC % V == 0, "records are whole 16-byte chunks");
  constexpr int CB = (kRing * NR / V + kThreads - 1) / kThreads;
  constexpr int CX = (kRing * NC / V + kThreads - 1) / kThreads;
  constexpr int CC = (NR / V + kThreads - 1) / kThreads;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads, h = tile - b * a.nheads, g = h / a.hpg;
  const float Ah = a.A[h], Dh = a.D[h];
  rs_meta* mp = a.meta + b;
  uint32_t* actr = a.arrive + static_cast<size_t>(b) * arrive_groups(a.nheads) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 2 ? RS_ERR_FULL : 0);
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, h, nck, len, nd);
    arr.finish(mp, actr, h, a.nheads, MetaOp::NonFlush, 0, nck, len, nd);
    return;
  }
  const int j = len + 1;
  const size_t bg = static_cast<size_t>(b) * a.ngroups + g;
  const TIN* inB = static_cast<const TIN*>(a.B) + bg * NR;
  const TIN* inC = static_cast<const TIN*>(a.C) + bg * NR;
  const TIN* inX = static_cast<const TIN*>(a.x) + static_cast<size_t>(tile) * NC;
  const TIN* inDt = static_cast<const TIN*>(a.dt) + tile;
  TIN* rB = static_cast<TIN*>(a.rB) + bg * kRing * NR;
  TIN* rC = static_cast<TIN*>(a.rC) + bg * kRing * NR;
  TIN* rX = static_cast<TIN*>(a.rx) + static_cast<size_t>(tile) * kRing * NC;
  TIN* rDt = static_cast<TIN*>(a.rdt) + static_cast<size_t>(tile) * kRing;
  // 1. buffer records into registers
  RegChunks<TIN, CB> cb;
  RegChunks<TIN, CX> cx;
  RegChunks<TIN, CC> cc;
  cb.load(EntrySrc<TIN>{rB, inB, 0, nck, len, NR}, j, NR);
  cx.load(EntrySrc<TIN>{rX, inX, 0, nck, len, NC}, j, NC);
  cc.load(EntrySrc<TIN>{inC, inC, 0, 0, 0, NR}, 1, NR);
  const int de = static_cast<int>(threadIdx.x) < j ? static_cast<int>(threadIdx.x) : j - 1;
  const float dtv = to_f(*(de < len ? rDt + ((nck + de) & (kRing - 1)) : inDt));
  // 2. the state tile, then the arrival count
  RawTile<RDF, E, NR, NC> raw;
  raw.issue(a.rd, tile);
  arr.arrive(actr, h, nck, len, nd);
  // 3. records to LDS, then the state-independent work
  cb.to_lds(&s.B[0][0], NR, j, NR);
  cx.to_lds(&s.X[0][0], NC, j, NC);
  cc.to_lds(s.C, NR, 1, NR);
  {
    // decays: thread e < 16 holds a_e = exp(dt_e A) (1 past the window); the
    // suffix products over its 16-lane row give the weights' decay
    // prod_{e<l<j} a_l and the checkpoint's L = prod_{l<j} a_l
    const int e = static_cast<int>(threadIdx.x);
    const float ae = e < j ? expf(dtv * Ah) : 1.0f;
    const float suf = row_suffix_prod16(ae);
    const float after = row_next16(suf);
    if (e < j) {
      s.dt[e] = dtv;
      s.a[e] = after;
    }
    if (e == 0) s.L = suf;
  }
  __syncthreads();
  {
    const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
    for (int e = grp; e < j; e += kThreads / 16) {
      float part = lds_dot16<NR>(&s.B[e][0], s.C, ln);
      part = group_sum16(part);
      if (ln == 0) s.w[e] = s.a[e] * s.dt[e] * part;
    }
  }
  __syncthreads();
  float buf = 0.0f;   // buffer part of y for column p = threadIdx.x
  if (static_cast<int>(threadIdx.x) < NC) {
    const int p = threadIdx.x;
    buf = Dh * s.X[j - 1][p];
    for (int e = 0; e < j; ++e) buf += s.w[e] * s.X[e][p];
  }
  // 4. the reduction over the state, y
  RegTile<E, NR, NC> H;
  raw.decode(H);
  tile_matvec<1>(H, s.C, NR, s.red, s.out);
  if (static_cast<int>(threadIdx.x) < NC) s.out[threadIdx.x] = s.L * s.out[threadIdx.x] + buf;
  __syncthreads();
  store_rows_nt(a.y + static_cast<size_t>(tile) * NC, s.out, NC);
  // 5. append the current record from its staged copy (exact: the values came from TIN)
  const int slot = static_cast<int>((nck + len) & (kRing - 1));
  store_row_as(rX + slot * NC, &s.X[j - 1][0], NC);
  if (threadIdx.x == 0) rDt[slot] = from_f<TIN>(s.dt[j - 1]);
  if (h % a.hpg == 0) {
    store_row_as(rB + slot * NR, &s.B[j - 1][0], NR);
    store_row_as(rC + slot * NR, s.C, NR);
  }
  arr.finish(mp, actr, h, a.nheads, MetaOp::NonFlush, 0, nck, len, nd);
}

template <typename TIN, int RDF, int NR, int NC>
__global__ __launch_bounds__(kThreads) void m2_nonflush_kernel(M2Args a) {
  __shared__ M2NfSmem<NR, NC> s;
  m2_nonflush_body<TIN, RDF, NR, NC>(a, s);
}

// ----------------------------------------------------------------------------
// non-flush step for FP16 / FP8 / NVFP4 reads: one wavefront per head, kHPB heads
// of one B/C group per workgroup. A low-precision tile (4.6 KiB in NVFP4) is
// smaller than the buffer records a head needs, so the group's B rows, C and
// the B.C dots are staged and computed once for kHPB heads, and each head's
// output is reduced inside its wavefront: lane l owns the 8 columns
// 8 (l mod 8) .. +7 of rows l/8 + 8k of the tile and of the held x rows l/8 and
// l/8 + 8, so the buffer term and D x join the lane's partial sums before one
// 3-step shuffle reduction over the 8 lanes that share those columns.
// ----------------------------------------------------------------------------
constexpr int kHPB = 4;

template <int NR, int NC>
struct alignas(16) M2WaveSmem {
  float B[kRing][NR];
  float C[NR];
  float bc[kRing];            // B_e . C_cur
  float w[kHPB][kRing];       // w_{j,e} dt_e (B_e . C_cur) per head
  float L[kHPB];
  // NVFP4 reads: each head's block scales, in the order the reduction reads
  // them: the scale of row 8 k + r, column block c at ((r (NC/16) + c) NR/8 + k),
  // so that a lane's scales (one row residue r and one block c, every k) are
  // one contiguous run
  alignas(16) uint8_t scl[kHPB][NR * NC / 16];
};

// FP8 and NVFP4 reads with bf16 records fit in 80 registers, which gives 6
// waves per SIMD instead of 5: more loads in flight for these short tiles.
template <typename TIN, int RDF, int NR, int NC>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu((RDF == FMT_F16 || sizeof(TIN) == 4) ? 1 : 6, 8)))
void m2_nonflush_wave_kernel(M2Args a) {
  static_assert(RDF == FMT_F16 || RDF == FMT_FP8 || RDF == FMT_NVFP4,
                "2-byte or smaller reads (an fp32 head needs 128 registers per lane here)");
  static_assert(NC == 64 && NR % 8 == 0, "8 lanes per 64-column row");
  constexpr int V = 16 / static_cast<int>(sizeof(TIN));
  constexpr int XCH = 8 / V;                 // 16-byte chunks per lane per x row (8 columns)
  constexpr int RPP = 8, PASSES = NR / RPP;   // tile rows per pass, passes per head
  constexpr int CB = (kRing * NR / V + kThreads - 1) / kThreads;
  constexpr int CC = (NR / V + kThreads - 1) / kThreads;
  __shared__ M2WaveSmem<NR, NC> s;
  const int nblk = a.nheads / kHPB;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);          // (sequence, head block)
  const int b = tile / nblk, hb = tile - b * nblk;
  // the wave index is uniform per wavefront: as a scalar, everything derived
  // from it (head, matrix, record pointers, D, matrix scale) stays in scalar
  // registers and its loads are scalar loads, which do not queue behind the tile
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int h = hb * kHPB + wave, g = (hb * kHPB) / a.hpg;
  rs_meta* mp = a.meta + b;
  uint32_t* actr = a.arrive + static_cast<size_t>(b) * arrive_groups(nblk) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 2 ? RS_ERR_FULL : 0);
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, hb, nck, len, nd);
    arr.finish(mp, actr, hb, nblk, MetaOp::NonFlush, 0, nck, len, nd);
    return;
  }
  const int j = len + 1;
  const size_t bg = static_cast<size_t>(b) * a.ngroups + g;
  const size_t mat = static_cast<size_t>(b) * a.nheads + h;
  const TIN* inB = static_cast<const TIN*>(a.B) + bg * NR;
  const TIN* inC = static_cast<const TIN*>(a.C) + bg * NR;
  const TIN* inX = static_cast<const TIN*>(a.x) + mat * NC;
  TIN* rB = static_cast<TIN*>(a.rB) + bg * kRing * NR;
  TIN* rC = static_cast<TIN*>(a.rC) + bg * kRing * NR;
  TIN* rX = static_cast<TIN*>(a.rx) + mat * kRing * NC;
  const size_t hdt = static_cast<size_t>(b) * a.nheads + hb * kHPB;   // first head of the block
  // 1. records into registers: group B rows and C (whole block), this head's x
  //    rows of entries lane/8 and lane/8 + 8 (8 columns), the block's dt
  RegChunks<TIN, CB> cb;
  RegChunks<TIN, CC> cc;
  cb.load(EntrySrc<TIN>{rB, inB, 0, nck, len, NR}, j, NR);
  cc.load(EntrySrc<TIN>{inC, inC, 0, 0, 0, NR}, 1, NR);
  const EntrySrc<TIN> xs{rX, inX, 0, nck, len, NC};
  const int ce = lane & 7, e0 = lane >> 3, e1 = e0 + 8;
  uint4 xr[2][XCH];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = q == 0 ? e0 : e1;
    const int ec = e < j ? e : j - 1;         // unconditional load from a valid entry
#pragma unroll
    for (int c = 0; c < XCH; ++c) xr[q][c] = *reinterpret_cast<const uint4*>(xs.at(ec) + ce * 8 + c * V);
  }
  // the block's dt and A with the records: a load issued after the tile would
  // return after all of it (in-order returns) and hold the first barrier there
  float dtv = 0.0f, Av = 0.0f;
  {
    const int t = threadIdx.x, hw = t >> 4, e = t & 15;
    const int ec = e < j ? e : j - 1;
    const TIN* rD = static_cast<const TIN*>(a.rdt) + (hdt + (hw < kHPB ? hw : 0)) * kRing;
    const TIN* iD = static_cast<const TIN*>(a.dt) + hdt + (hw < kHPB ? hw : 0);
    dtv = to_f(*(ec < len ? rD + ((nck + ec) & (kRing - 1)) : iD));
    Av = a.A[hb * kHPB + (hw < kHPB ? hw : 0)];
  }
  const float Dh = a.D[h];                     // per-wave values ahead of the tile too
  const float ms = mat_scale<RDF>(a.rd, mat);   // FP8 / NVFP4 matrix scale
  // 2. this head's tile, then the arrival count
  // NVFP4: the head's block scales come as one 4- or 8-byte load per lane
  // (not a byte load per chunk) and go to LDS with the records; each chunk's
  // scale is read back from there when it is decoded
  constexpr int SPL = NR * NC / 16 / 64;       // scale bytes per lane
  static_assert(RDF != FMT_NVFP4 || SPL == 4 || SPL == 8, "whole-lane scale loads");
  uint2 scv = make_uint2(0u, 0u);
  Raw<RDF, 8> raw[PASSES];
  __builtin_amdgcn_sched_barrier(0);           // the record loads stay ahead of the tile
  if constexpr (RDF == FMT_NVFP4) {
    const uint8_t* sp = a.rd.nv_scale + mat * (NR * NC / 16) + lane * SPL;
    if constexpr (SPL == 8) scv = nt_load(reinterpret_cast<const uint2*>(sp));
    else scv.x = nt_load(reinterpret_cast<const uint32_t*>(sp));
  }
  // the head's tile from a scalar base plus one 32-bit lane offset, so that
  // consecutive passes differ only in the load's immediate offset
  constexpr int RB = RDF == FMT_F16 ? 2 * NC : RDF == FMT_FP8 ? NC : NC / 2;   // bytes per tile row
  const uint8_t* tb = static_cast<const uint8_t*>(a.rd.data) + mat * static_cast<size_t>(NR * RB);
  const uint32_t lo = static_cast<uint32_t>((lane >> 3) * RB + ce * (8 * RB / NC));
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const uint8_t* p = tb + lo + k * (RPP * RB);
    if constexpr (RDF == FMT_NVFP4) {
      raw[k].v = nt_load(reinterpret_cast<const uint32_t*>(p));
      raw[k].s = 0u;
    } else if constexpr (RDF == FMT_FP8) {
      raw[k].v = nt_load(reinterpret_cast<const uint2*>(p));
    } else {
      raw[k].v = nt_load(reinterpret_cast<const uint4*>(p));
    }
  }
  arr.arrive(actr, hb, nck, len, nd);
  // 3. records to LDS; dots, decays and weights (state-independent)
  cb.to_lds(&s.B[0][0], NR, j, NR);
  cc.to_lds(s.C, NR, 1, NR);
  if constexpr (RDF == FMT_NVFP4) {
    // lane's scale bytes i: row (SPL lane + i) / (NC/16), block (SPL lane + i) mod (NC/16)
    constexpr int NB = NC / 16;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int idx = lane * SPL + i, row = idx / NB, blk = idx - row * NB;
      const uint32_t word = i < 4 ? scv.x : scv.y;
      s.scl[wave][((row & (RPP - 1)) * NB + blk) * PASSES + row / RPP] =
          static_cast<uint8_t>(word >> (8 * (i & 3)));
    }
  }
  __syncthreads();
  {
    const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
    if (grp < j) {
      float part = lds_dot16<NR>(&s.B[grp][0], s.C, ln);
      part = group_sum16(part);
      if (ln == 0) s.bc[grp] = part;
    }
  }
  // decays in registers: thread 16 hw + e holds a_e = exp(dt_e A) of head hw
  // (1 past the window); the row's suffix products give the weights'
  // decay prod_{e<l<j} a_l and the checkpoint's L = prod_{l<j} a_l
  const int e_of = threadIdx.x & 15;
  const float ae = threadIdx.x < kHPB * 16 && e_of < j ? expf(dtv * Av) : 1.0f;
  const float suf = row_suffix_prod16(ae);
  const float after = row_next16(suf);
  __syncthreads();
  if (threadIdx.x < kHPB * 16) {
    const int hw = threadIdx.x >> 4;
    if (e_of < j) s.w[hw][e_of] = after * dtv * s.bc[e_of];
    if (e_of == 0) s.L[hw] = suf;
  }
  __syncthreads();
  // 4. this head's output inside its wavefront; a chunk's elements share one
  //    row weight C_n, so its block scale joins that weight and the matrix
  //    scale joins L (one multiply per chunk instead of one per element)
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  // NVFP4: this lane's PASSES block scales as one LDS read, decoded two per
  // conversion (exactly, as E4M3 values) as the passes reach them
  static_assert(RDF != FMT_NVFP4 || PASSES % 4 == 0, "whole words of scale bytes");
  uint32_t sw[RDF == FMT_NVFP4 ? PASSES / 4 : 1];
  if constexpr (RDF == FMT_NVFP4) {
    const uint8_t* sp = &s.scl[wave][((lane >> 3) * (NC / 16) + (ce >> 1)) * PASSES];
    if constexpr (PASSES == 16) {
      const uint4 q = *reinterpret_cast<const uint4*>(sp);
      sw[0] = q.x; sw[1] = q.y; sw[2] = q.z; sw[3] = q.w;
    } else {
#pragma unroll
      for (int m = 0; m < PASSES / 4; ++m) sw[m] = reinterpret_cast<const uint32_t*>(sp)[m];
    }
  }
  f32x2 bpair = {1.0f, 1.0f};
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    float t[8];
    decode_codes8<RDF>(raw[k], t);
    if constexpr (RDF == FMT_NVFP4) {
      if (k % 4 == 0) bpair = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[k / 4], 1.0f, false);   // bytes 0, 1
      if (k % 4 == 2) bpair = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[k / 4], 1.0f, true);    // bytes 2, 3
    }
    const float cr = (k % 2 == 0 ? bpair.x : bpair.y) * s.C[k * RPP + (lane >> 3)];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += t[i] * cr;
  }
  const float L = s.L[wave] * ms;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] *= L;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = q == 0 ? e0 : e1;
    float xv[8];
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
      // entries past the window contribute 0 (their rows, copies of the last entry's, are cleared)
      const uint4 xw = e < j ? xr[q][c] : make_uint4(0u, 0u, 0u, 0u);
      unpack16(xw, static_cast<const TIN*>(nullptr), xv + c * V);
    }
    const float we = e < j ? s.w[wave][e] + (e == j - 1 ? Dh : 0.0f) : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += we * xv[i];
  }
  int col;
  const float yv = transpose_sum8(acc, col);
  nt_store(yv, a.y + mat * NC + ce * 8 + col);
  // 5. append the current record (bit copies)
  const int slot = static_cast<int>((nck + len) & (kRing - 1));
  if (lane < NC / V) reinterpret_cast<uint4*>(rX + slot * NC)[lane] = reinterpret_cast<const uint4*>(inX)[lane];
  if (lane == 0) static_cast<TIN*>(a.rdt)[mat * kRing + slot] = static_cast<const TIN*>(a.dt)[mat];
  if (wave == 0 && (hb * kHPB) % a.hpg == 0) {
    if (lane < NR / V) {
      reinterpret_cast<uint4*>(rB + slot * NR)[lane] = reinterpret_cast<const uint4*>(inB)[lane];
      reinterpret_cast<uint4*>(rC + slot * NR)[lane] = reinterpret_cast<const uint4*>(inC)[lane];
    }
  }
  arr.finish(mp, actr, hb, nblk, MetaOp::NonFlush, 0, nck, len, nd);
}

// ----------------------------------------------------------------------------
// fold body shared by the flush step and the commit fold
// H <- l_m H + sum_e B_e xt_e^T with xt_e = w_{m,e} dt_e x_e (entries staged)
// ----------------------------------------------------------------------------
// Coefficients of the fold into LDS: L = l_m and xt_e = w_{m,e} dt_e x_e.
// Barriers inside; all threads must call.
// The decay products come from suffix products over one 16-lane row (lane e
// holds a_e, 1 from m on): w_{m,e} is the product from e + 1 on, l_m the
// row's whole product.
template <typename SM>
__device__ __forceinline__ void fold_coeffs(SM& s, int m) {
  constexpr int NC = sizeof(s.X[0]) / sizeof(float);
  static_assert(kRing == 16, "one DPP row holds the window");
  if (threadIdx.x < 16) {
    const int e = threadIdx.x;
    const float suf = row_suffix_prod16(e < m ? s.a[e] : 1.0f);   // prod_{e <= l < m} a_l
    const float w = row_next16(suf);                                // prod_{e < l < m} a_l
    if (e < m) s.w[0][e] = w * s.dt[e];
    if (e == 0) s.L[0] = suf;
  }
  __syncthreads();
  static_assert(NC % 4 == 0, "float4 rows");
  for (int idx = threadIdx.x; idx < m * (NC / 4); idx += kThreads) {
    const int e = idx / (NC / 4), p = 4 * (idx - e * (NC / 4));
    const float w = s.w[0][e];
    const float4 x = *reinterpret_cast<const float4*>(&s.X[e][p]);
    *reinterpret_cast<float4*>(&s.xt[e][p]) = make_float4(w * x.x, w * x.y, w * x.z, w * x.w);
  }
  __syncthreads();
}

template <int E, int NR, int NC, typename SM>
__device__ __forceinline__ void fold_tile(RegTile<E, NR, NC>& H, SM& s, int m) {
  fold_coeffs(s, m);
  const float L = s.L[0];
  const int c0 = RegTile<E, NR, NC>::col0();
#pragma unroll
  for (int k = 0; k < RegTile<E, NR, NC>::P; ++k)
#pragma unroll
    for (int i = 0; i < E; ++i) H.v[k][i] *= L;
  for (int e = 0; e < m; ++e) {
    float xt[E];
#pragma unroll
    for (int i = 0; i < E; ++i) xt[i] = s.xt[e][c0 + i];
#pragma unroll
    for (int k = 0; k < RegTile<E, NR, NC>::P; ++k) {
      const int row = RegTile<E, NR, NC>::row(k);
      if (row < NR) {
        const float br = s.B[e][row];
#pragma unroll
        for (int i = 0; i < E; ++i) H.v[k][i] += br * xt[i];
      }
    }
  }
}

// Store the folded tile in the checkpoint format, and the NVFP4 read copy of
// the stored values when asked. For an fp32 checkpoint the read copy's maximum
// is reduced before the checkpoint's stores go out: the reduction's workgroup
// barriers would otherwise wait for those 32 KiB of stores (measured 476 ->
// 454 us per flush at batch 256). For fp16 and fp8 checkpoints the stores go
// out first and overlap the requantisation (reordering those measured slower).
template <int CKF, bool RC, int E, int NR, int NC>
__device__ __forceinline__ void store_folded(const M2Args& a, size_t tile, RegTile<E, NR, NC>& H, float* s4) {
  if constexpr (RC && CKF == FMT_F32) {
    if (a.fuse_rc) {
      const float amax = tile_absmax(H, s4);
      tile_store<FMT_F32>(a.ck, tile, H, s4);
      tile_store_nvfp4(a.rc, tile, H, amax);
      return;
    }
  }
  tile_store<CKF>(a.ck, tile, H, s4);
  if constexpr (RC) {
    if (a.fuse_rc) {
      tile_round_trip<CKF>(H, s4);
      tile_store<FMT_NVFP4>(a.rc, tile, H, s4);
    }
  }
}

// The fold, the output matvec and the store of the flush and commit-fold, on
// one of two tile layouts: the streaming layout (each thread owns E
// consecutive columns of rows spaced a pass apart; rank-m update on fp32 FMAs)
// or the matrix-core layout of rs_mtile.h (rank-m update on
// v_mfma_f32_16x16x4f32; each lane owns 16 consecutive columns of a row).
template <int CKF, bool RC, int NR, int NC>
struct ValuFold {
  static constexpr int E = CKF == FMT_F32 ? 4 : 8;
  using Raw = RawTile<CKF, E, NR, NC>;
  using Tile = RegTile<E, NR, NC>;
  template <typename SM>
  __device__ __forceinline__ static void fold(const Raw& raw, Tile& H, SM& s, int m) {
    raw.decode(H);
    fold_tile(H, s, m);
  }
  __device__ __forceinline__ static void matvec(const Tile& H, const float* w, float* red, float* out) {
    tile_matvec<1>(H, w, NR, red, out);
  }
  __device__ __forceinline__ static void store(const M2Args& a, size_t tile, Tile& H, float* s4) {
    store_folded<CKF, RC>(a, tile, H, s4);
  }
};

template <int CKF, bool RC, int NR, int NC>
struct MfmaFold {
  using Raw = MRaw<CKF, NR, NC>;
  using Tile = MTile<NR, NC>;
  // the decay product l_m is applied as the tile is decoded
  template <typename SM>
  __device__ __forceinline__ static void fold(const Raw& raw, Tile& H, SM& s, int m) {
    fold_coeffs(s, m);
    raw.decode(H, s.L[0]);
    mtile_rank_update(H, &s.B[0][0], NR, &s.xt[0][0], NC, m);
  }
  __device__ __forceinline__ static void matvec(const Tile& H, const float* w, float* red, float* out) {
    mtile_matvec(H, w, red, out);
  }
  // as store_folded: for an fp32 checkpoint the copy's maximum is reduced
  // before the checkpoint's stores go out
  __device__ __forceinline__ static void store(const M2Args& a, size_t tile, Tile& H, float* s4) {
    if constexpr (RC && CKF == FMT_F32) {
      if (a.fuse_rc) {
        const float amax = mtile_absmax(H, s4);
        mtile_store<FMT_F32>(a.ck, tile, H, s4);
        mtile_store<FMT_NVFP4>(a.rc, tile, H, s4, amax);
        return;
      }
    }
    mtile_store<CKF>(a.ck, tile, H, s4);
    if constexpr (RC) {
      if (a.fuse_rc) {
        mtile_round_trip<CKF>(H, s4);
        mtile_store<FMT_NVFP4>(a.rc, tile, H, s4);
      }
    }
  }
};

// Which layout folds a (format, shape), by measurement at batch 256 on the
// 128 x 64 state (flush times, streaming vs matrix-core layout): fp32 374.9
// vs 437.1 us and fp32 + NVFP4 copy 455.9 vs 515.4 (the fp32 flush is bound
// by its traffic, which the streaming layout moves in whole 1 KiB rows per
// instruction); fp16 214.1 vs 240.9; fp16 + copy 284.0 vs 271.2; fp8 246.7
// vs 199.7; fp8 + copy 358.5 vs 341.5; uniform NVFP4 261.0 vs 210.1 (these
// are bound by the fold's arithmetic on the streaming layout).
template <int CKF, bool RC, int NR, int NC>
constexpr bool kMfmaFold =
    NR % 64 == 0 && NC % 64 == 0 && (CKF == FMT_FP8 || CKF == FMT_NVFP4 || (CKF == FMT_F16 && RC));

template <int CKF, bool RC, int NR, int NC>
using FoldOps = typename std::conditional<kMfmaFold<CKF, RC, NR, NC>, MfmaFold<CKF, RC, NR, NC>,
                                          ValuFold<CKF, RC, NR, NC>>::type;

// ----------------------------------------------------------------------------
// flush step: fold len stored entries + the current token, write once, y
// ----------------------------------------------------------------------------
template <int NR, int NC>
using M2FlSmem = M2Smem<NR, NC, kRing, 1, true>;

template <typename TIN, int CKF, bool RC, int NR, int NC>
__device__ __forceinline__ void m2_flush_body(const M2Args& a, M2FlSmem<NR, NC>& s) {
  using Ops = FoldOps<CKF, RC, NR, NC>;
  constexpr int V = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NR % V == 0 && NC % V == 0, "records are whole 16-byte chunks");
  constexpr int CB = (kRing * NR / V + kThreads - 1) / kThreads;
  constexpr int CX = (kRing * NC / V + kThreads - 1) / kThreads;
  constexpr int CC = (NR / V + kThreads - 1) / kThreads;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads, h = tile - b * a.nheads, g = h / a.hpg;
  const float Ah = a.A[h], Dh = a.D[h];   // before the tile: a load behind it would wait for all of it
  // The matrix-core folds take the checkpoint tile first (its address does not
  // depend on the counters, so it is in flight while they are read); the
  // streaming folds take it after the records, which then arrive first and are
  // staged while the tile streams in. Measured at batch 256 on the 128 x 64
  // state (flush us, records first -> tile first): fp8 195.2 -> 189.3, NVFP4
  // 214.2 -> 199.1, fp8 + copy 336.5 -> 319.8, fp16 + copy 269.1 -> 256.8;
  // fp32 + copy 454.4 -> 464.0, fp16 183.2 -> 186.9.
  constexpr bool kTileFirst = kMfmaFold<CKF, RC, NR, NC>;
  typename Ops::Raw raw;
  if constexpr (kTileFirst) {
    raw.issue(a.ck, tile);
    __builtin_amdgcn_sched_barrier(0);
  }
  rs_meta* mp = a.meta + b;
  uint32_t* actr = a.arrive + static_cast<size_t>(b) * arrive_groups(a.nheads) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 1 ? RS_ERR_FULL : 0);
  const int m = len + 1;
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, h, nck, len, nd);
  } else {
    const size_t bg = static_cast<size_t>(b) * a.ngroups + g;
    const TIN* inB = static_cast<const TIN*>(a.B) + bg * NR;
    const TIN* inC = static_cast<const TIN*>(a.C) + bg * NR;
    const TIN* inX = static_cast<const TIN*>(a.x) + static_cast<size_t>(tile) * NC;
    const TIN* inDt = static_cast<const TIN*>(a.dt) + tile;
    const TIN* rB = static_cast<const TIN*>(a.rB) + bg * kRing * NR;
    const TIN* rX = static_cast<const TIN*>(a.rx) + static_cast<size_t>(tile) * kRing * NC;
    const TIN* rDt = static_cast<const TIN*>(a.rdt) + static_cast<size_t>(tile) * kRing;
    // records into registers (then the state tile, unless it went first), then records to LDS
    RegChunks<TIN, CB> cb;
    RegChunks<TIN, CX> cx;
    RegChunks<TIN, CC> cc;
    cb.load(EntrySrc<TIN>{rB, inB, 0, nck, len, NR}, m, NR);
    cx.load(EntrySrc<TIN>{rX, inX, 0, nck, len, NC}, m, NC);
    cc.load(EntrySrc<TIN>{inC, inC, 0, 0, 0, NR}, 1, NR);
    const int de = static_cast<int>(threadIdx.x) < m ? static_cast<int>(threadIdx.x) : m - 1;
    const float dtv = to_f(*EntrySrc<TIN>{rDt, inDt, 0, nck, len, 1}.at(de));
    if constexpr (!kTileFirst) raw.issue(a.ck, tile);
    arr.arrive(actr, h, nck, len, nd);
    cb.to_lds(&s.B[0][0], NR, m, NR);
    cx.to_lds(&s.X[0][0], NC, m, NC);
    cc.to_lds(&s.Cw[0][0], NR, 1, NR);
    if (static_cast<int>(threadIdx.x) < m) {
      s.dt[threadIdx.x] = dtv;
      s.a[threadIdx.x] = expf(dtv * Ah);
    }
    __syncthreads();
    typename Ops::Tile H;
    Ops::fold(raw, H, s, m);
    Ops::matvec(H, &s.Cw[0][0], s.red, s.out);
    for (int p = threadIdx.x; p < NC; p += kThreads)
      a.y[static_cast<size_t>(tile) * NC + p] = s.out[p] + Dh * s.X[m - 1][p];
    Ops::store(a, tile, H, s.s4);
  }
  arr.finish(mp, actr, h, a.nheads, MetaOp::Flush, 0, nck, len, nd);
}

template <typename TIN, int CKF, bool RC, int NR, int NC>
__global__ __launch_bounds__(kThreads) void m2_flush_kernel(M2Args a) {
  __shared__ M2FlSmem<NR, NC> s;
  m2_flush_body<TIN, CKF, RC, NR, NC>(a, s);
}

// ----------------------------------------------------------------------------
// self-scheduling step (continuous batching): each sequence takes the flush
// when its buffer is full and a non-flush step otherwise, in one launch, so
// sequences at different fills share a batch and the flush work spreads over
// steps. The branch is uniform per workgroup (one sequence, one head).
// ----------------------------------------------------------------------------
template <int NR, int NC>
union M2AutoSmem {
  M2NfSmem<NR, NC> nf;
  M2FlSmem<NR, NC> fl;
};

template <typename TIN, int CKF, bool RC, int NR, int NC>
__global__ __launch_bounds__(kThreads) void m2_auto_kernel(M2Args a) {
  constexpr int RDF = RC ? FMT_NVFP4 : CKF;   // what a non-flush step reads
  __shared__ M2AutoSmem<NR, NC> s;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads;
  if (a.meta[b].len == kRing - 1) m2_flush_body<TIN, CKF, RC, NR, NC>(a, s.fl);
  else m2_nonflush_body<TIN, RDF, NR, NC>(a, s.nf);
}

// ----------------------------------------------------------------------------
// speculative append (ReplaySSM): K verify outputs from checkpoint + buffer +
// drafts, drafts written to the ring, no state write
// ----------------------------------------------------------------------------
template <typename TIN, int RDF, int NR, int NC, int KQ>
__global__ __launch_bounds__(kThreads) void m2_spec_append_kernel(M2Args a) {
  constexpr int E = (RDF == FMT_F32) ? 4 : 8;
  constexpr int V = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NR % V == 0 && NC % V == 0, "records are whole 16-byte chunks");
  constexpr int CB = (kRing * NR / V + kThreads - 1) / kThreads;
  constexpr int CX = (kRing * NC / V + kThreads - 1) / kThreads;
  constexpr int CC = (KQ * NR / V + kThreads - 1) / kThreads;
  __shared__ M2Smem<NR, NC, kRing, KQ, false> s;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads, h = tile - b * a.nheads, g = h / a.hpg;
  const int K = a.K;
  const float Ah = a.A[h];
  rs_meta* mp = a.meta + b;
  uint32_t* actr = a.arrive + static_cast<size_t>(b) * arrive_groups(a.nheads) * kArriveStride;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = (nd != 0 || len + K > kRing) ? RS_ERR_OVERFLOW : 0;
  Arrival arr;
  if (errbit != 0) {
    arr.arrive(actr, h, nck, len, nd);
  } else {
    const size_t bg = static_cast<size_t>(b) * a.ngroups + g;
    const size_t gstride = static_cast<size_t>(a.batch) * a.ngroups * NR;   // between drafts (B, C)
    const size_t xstride = static_cast<size_t>(a.batch) * a.nheads * NC;    // between drafts (x)
    const size_t dstride = static_cast<size_t>(a.batch) * a.nheads;         // between drafts (dt)
    const TIN* inB = static_cast<const TIN*>(a.B) + bg * NR;
    const TIN* inC = static_cast<const TIN*>(a.C) + bg * NR;
    const TIN* inX = static_cast<const TIN*>(a.x) + static_cast<size_t>(tile) * NC;
    const TIN* inDt = static_cast<const TIN*>(a.dt) + tile;
    TIN* rB = static_cast<TIN*>(a.rB) + bg * kRing * NR;
    TIN* rC = static_cast<TIN*>(a.rC) + bg * kRing * NR;
    TIN* rX = static_cast<TIN*>(a.rx) + static_cast<size_t>(tile) * kRing * NC;
    TIN* rDt = static_cast<TIN*>(a.rdt) + static_cast<size_t>(tile) * kRing;
    const int n = len + K;
    // records into registers, then the state tile, then records to LDS
    RegChunks<TIN, CB> cb;
    RegChunks<TIN, CX> cx;
    RegChunks<TIN, CC> cc;
    cb.load(EntrySrc<TIN>{rB, inB, gstride, nck, len, NR}, n, NR);
    cx.load(EntrySrc<TIN>{rX, inX, xstride, nck, len, NC}, n, NC);
    cc.load(EntrySrc<TIN>{inC, inC, gstride, 0, 0, NR}, K, NR);
    const int de = static_cast<int>(threadIdx.x) < n ? static_cast<int>(threadIdx.x) : n - 1;
    const float dtv = to_f(*EntrySrc<TIN>{rDt, inDt, dstride, nck, len, 1}.at(de));
    RawTile<RDF, E, NR, NC> raw;
    raw.issue(a.rd, tile);
    arr.arrive(actr, h, nck, len, nd);
    cb.to_lds(&s.B[0][0], NR, n, NR);
    cx.to_lds(&s.X[0][0], NC, n, NC);
    cc.to_lds(&s.Cw[0][0], NR, K, NR);
    for (int idx = K * NR + threadIdx.x; idx < KQ * NR; idx += kThreads) (&s.Cw[0][0])[idx] = 0.0f;
    if (static_cast<int>(threadIdx.x) < n) {
      s.dt[threadIdx.x] = dtv;
      s.a[threadIdx.x] = expf(dtv * Ah);
    }
    __syncthreads();
    output_weights(s, len + 1, K);
    RegTile<E, NR, NC> H;
    raw.decode(H);
    tile_matvec<KQ>(H, &s.Cw[0][0], NR, s.red, s.out);
    const float Dh = a.D[h];
    for (int idx = threadIdx.x; idx < K * NC; idx += kThreads) {   // in place: s.out[idx] is this thread's
      const int d = idx / NC, p = idx - d * NC;
      const int J = len + d + 1;
      float yv = s.L[d] * s.out[idx];
      for (int e = 0; e < J; ++e) yv += s.w[d][e] * s.X[e][p];
      s.out[idx] = yv + Dh * s.X[J - 1][p];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < K * NC / 4; i += kThreads) {
      const int d = i / (NC / 4), c = i - d * (NC / 4);
      const float* o = &s.out[d * NC + 4 * c];
      nt_store(make_float4(o[0], o[1], o[2], o[3]),
               reinterpret_cast<float4*>(a.y + d * xstride + static_cast<size_t>(tile) * NC) + c);
    }
    // drafts into the ring from their staged copies (bit copies: the values came from TIN)
    const auto draft_slot = [&](int d) { return static_cast<int>((nck + len + d) & (kRing - 1)); };
    store_rows_as(rX, &s.X[len][0], NC, K, NC, draft_slot);
    if (static_cast<int>(threadIdx.x) < K) rDt[draft_slot(threadIdx.x)] = from_f<TIN>(s.dt[len + threadIdx.x]);
    if (h % a.hpg == 0) {
      store_rows_as(rB, &s.B[len][0], NR, K, NR, draft_slot);
      store_rows_as(rC, &s.Cw[0][0], NR, K, NR, draft_slot);
    }
  }
  arr.finish(mp, actr, h, a.nheads, MetaOp::Append, K, nck, len, nd);
}

// ----------------------------------------------------------------------------
// speculative commit (ReplaySSM): the counter part and its fold list are built
// by commit_meta (rs_commit.hip); here the listed sequences are folded.
// ----------------------------------------------------------------------------
// part 2: fold the listed sequences' committed entries, one head per work
// item, over a fixed grid (every workgroup leaves when the list is done)
template <typename TIN, int CKF, bool RC, int NR, int NC>
__global__ __launch_bounds__(kThreads) void m2_commit_fold_kernel(M2Args a) {
  using Ops = FoldOps<CKF, RC, NR, NC>;
  constexpr int V = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NR % V == 0 && NC % V == 0, "records are whole 16-byte chunks");
  constexpr int CB = (kRing * NR / V + kThreads - 1) / kThreads;
  constexpr int CX = (kRing * NC / V + kThreads - 1) / kThreads;
  __shared__ M2Smem<NR, NC, kRing, 1, true> s;
  const int total = *a.work_count * a.nheads;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const FoldItem it = a.work[item / a.nheads];
    const int h = item - (item / a.nheads) * a.nheads;
    const int b = it.b, g = h / a.hpg, m = it.m;
    const size_t tile = static_cast<size_t>(b) * a.nheads + h;
    const size_t bg = static_cast<size_t>(b) * a.ngroups + g;
    const TIN* rB = static_cast<const TIN*>(a.rB) + bg * kRing * NR;
    const TIN* rX = static_cast<const TIN*>(a.rx) + tile * kRing * NC;
    const TIN* rDt = static_cast<const TIN*>(a.rdt) + tile * kRing;
    // records into registers, then the state tile, then records to LDS
    RegChunks<TIN, CB> cb;
    RegChunks<TIN, CX> cx;
    cb.load(EntrySrc<TIN>{rB, rB, 0, it.nck, m, NR}, m, NR);
    cx.load(EntrySrc<TIN>{rX, rX, 0, it.nck, m, NC}, m, NC);
    const int de = static_cast<int>(threadIdx.x) < m ? static_cast<int>(threadIdx.x) : m - 1;
    const float dtv = to_f(*EntrySrc<TIN>{rDt, rDt, 0, it.nck, m, 1}.at(de));
    const float Ah = a.A[h];   // before the tile: a load behind it would wait for all of it
    typename Ops::Raw raw;
    raw.issue(a.ck, tile);
    cb.to_lds(&s.B[0][0], NR, m, NR);
    cx.to_lds(&s.X[0][0], NC, m, NC);
    if (static_cast<int>(threadIdx.x) < m) {
      s.dt[threadIdx.x] = dtv;
      s.a[threadIdx.x] = expf(dtv * Ah);
    }
    __syncthreads();
    typename Ops::Tile H;
    Ops::fold(raw, H, s, m);
    Ops::store(a, tile, H, s.s4);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------
// snapshot baseline: step the live state through K drafts, write each state
// to snap[d], K outputs; the live state is not written here
// ----------------------------------------------------------------------------
template <typename TIN, int NR, int NC, int KMAX>
__global__ __launch_bounds__(kThreads) void m2_conv_spec_kernel(M2Args a) {
  constexpr int E = 4;
  __shared__ M2Smem<NR, NC, KMAX, KMAX, false> s;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads, h = tile - b * a.nheads, g = h / a.hpg;
  const int K = a.K;
  constexpr int V = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NR % V == 0 && NC % V == 0, "records are whole 16-byte chunks");
  constexpr int CB = (KMAX * NR / V + kThreads - 1) / kThreads;
  constexpr int CX = (KMAX * NC / V + kThreads - 1) / kThreads;
  const size_t bg = static_cast<size_t>(b) * a.ngroups + g;
  const size_t gstride = static_cast<size_t>(a.batch) * a.ngroups * NR;
  const size_t xstride = static_cast<size_t>(a.batch) * a.nheads * NC;
  const size_t dstride = static_cast<size_t>(a.batch) * a.nheads;
  const TIN* inB = static_cast<const TIN*>(a.B) + bg * NR;
  const TIN* inC = static_cast<const TIN*>(a.C) + bg * NR;
  const TIN* inX = static_cast<const TIN*>(a.x) + static_cast<size_t>(tile) * NC;
  const TIN* inDt = static_cast<const TIN*>(a.dt) + tile;
  // the drafts' inputs into registers, then the state, then the inputs to LDS
  RegChunks<TIN, CB> cb, cc;
  RegChunks<TIN, CX> cx;
  cb.load(EntrySrc<TIN>{inB, inB, gstride, 0, 0, NR}, K, NR);
  cc.load(EntrySrc<TIN>{inC, inC, gstride, 0, 0, NR}, K, NR);
  cx.load(EntrySrc<TIN>{inX, inX, xstride, 0, 0, NC}, K, NC);
  const int de = static_cast<int>(threadIdx.x) < K ? static_cast<int>(threadIdx.x) : K - 1;
  const float dtv = to_f(inDt[de * dstride]);
  const float Ah = a.A[h];
  RawTile<FMT_F32, E, NR, NC> raw;
  raw.issue(a.ck, tile);
  cb.to_lds(&s.B[0][0], NR, K, NR);
  cc.to_lds(&s.Cw[0][0], NR, K, NR);
  cx.to_lds(&s.X[0][0], NC, K, NC);
  if (static_cast<int>(threadIdx.x) < K) {
    s.dt[threadIdx.x] = dtv;
    s.a[threadIdx.x] = expf(dtv * Ah);
  }
  __syncthreads();
  RegTile<E, NR, NC> H;
  raw.decode(H);
  const int c0 = RegTile<E, NR, NC>::col0();
  const float Dh = a.D[h];
  const size_t snap_stride = static_cast<size_t>(a.batch) * a.nheads;   // matrices per snapshot
  for (int d = 0; d < K; ++d) {
    const float decay = s.a[d];
    float dtx[E];
#pragma unroll
    for (int i = 0; i < E; ++i) dtx[i] = s.dt[d] * s.X[d][c0 + i];
#pragma unroll
    for (int k = 0; k < RegTile<E, NR, NC>::P; ++k) {
      const int row = RegTile<E, NR, NC>::row(k);
      if (row < NR) {
        const float br = s.B[d][row];
#pragma unroll
        for (int i = 0; i < E; ++i) H.v[k][i] = decay * H.v[k][i] + dtx[i] * br;
      }
    }
    StateBuf sn{a.snap, nullptr, nullptr};
    tile_store<FMT_F32>(sn, d * snap_stride + tile, H, s.s4);
    tile_matvec<1>(H, &s.Cw[d][0], NR, s.red, s.out);
    for (int p = threadIdx.x; p < NC; p += kThreads)
      a.y[d * xstride + static_cast<size_t>(tile) * NC + p] = s.out[p] + Dh * s.X[d][p];
  }
}

// snapshot baseline commit: live <- snap[k-1] for 1 <= k <= max_draft
template <int NR, int NC>
__global__ __launch_bounds__(kThreads) void m2_restore_kernel(M2Args a) {
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / a.nheads;
  const int k = a.accepted[b];
  if (k < 1 || k > a.kmax) return;
  const size_t snap_stride = static_cast<size_t>(a.batch) * a.nheads;
  const float4* src = reinterpret_cast<const float4*>(a.snap + ((k - 1) * snap_stride + tile) * NR * NC);
  float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.ck.data) + static_cast<size_t>(tile) * NR * NC);
  for (int i = threadIdx.x; i < NR * NC / 4; i += kThreads) nt_store(nt_load(src + i), dst + i);
}

// ----------------------------------------------------------------------------
// standalone read-copy quantizer: NVFP4 copy of the stored checkpoint
// ----------------------------------------------------------------------------
// (an fp32 checkpoint streams four columns per thread, the layout whose
// loads cover whole rows; the other formats' chunks are eight elements)
template <int CKF, int NR, int NC>
__global__ __launch_bounds__(kThreads) void requant_kernel(StateBuf ck, StateBuf rc) {
  constexpr int E = CKF == FMT_F32 ? 4 : 8;
  __shared__ float s4[4];
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  RawTile<CKF, E, NR, NC> raw;
  raw.issue(ck, tile);
  RegTile<E, NR, NC> H;
  raw.decode(H);
  tile_store<FMT_NVFP4>(rc, tile, H, s4);
}

// ----------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------

template <int NR, int NC>
struct M2Shape {
  template <typename TIN>
  static void conv(const M2Args& a, int grid, hipStream_t st) {
    m2_conv_kernel<TIN, NR, NC><<<grid, kThreads, 0, st>>>(a);
  }
  template <typename TIN>
  static void nonflush(const M2Args& a, int rdf, int grid, hipStream_t st) {
    if constexpr (NC == 64 && NR % 8 == 0) {
      // fp32 reads keep the 256-thread tile kernel: a whole fp32 head per wavefront
      // needs 170 registers per lane, 2 waves per SIMD, and measured 270 vs 177 us
      if (rdf != FMT_F32 && a.hpg % kHPB == 0) {
        const int g = grid / kHPB;   // one workgroup per kHPB heads
        if (rdf == FMT_F16) m2_nonflush_wave_kernel<TIN, FMT_F16, NR, NC><<<g, kThreads, 0, st>>>(a);
        else if (rdf == FMT_FP8) m2_nonflush_wave_kernel<TIN, FMT_FP8, NR, NC><<<g, kThreads, 0, st>>>(a);
        else m2_nonflush_wave_kernel<TIN, FMT_NVFP4, NR, NC><<<g, kThreads, 0, st>>>(a);
        return;
      }
    }
    switch (rdf) {
      case FMT_F32: m2_nonflush_kernel<TIN, FMT_F32, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_F16: m2_nonflush_kernel<TIN, FMT_F16, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_FP8: m2_nonflush_kernel<TIN, FMT_FP8, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      default: m2_nonflush_kernel<TIN, FMT_NVFP4, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
    }
  }
  template <typename TIN, bool RC>
  static void flush_rc(const M2Args& a, int ckf, int grid, hipStream_t st) {
    switch (ckf) {
      case FMT_F32: m2_flush_kernel<TIN, FMT_F32, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_F16: m2_flush_kernel<TIN, FMT_F16, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_FP8: m2_flush_kernel<TIN, FMT_FP8, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      default: m2_flush_kernel<TIN, FMT_NVFP4, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
    }
  }
  template <typename TIN>
  static void flush(const M2Args& a, int ckf, bool rc, int grid, hipStream_t st) {
    if (rc) flush_rc<TIN, true>(a, ckf, grid, st);
    else flush_rc<TIN, false>(a, ckf, grid, st);
  }
  template <typename TIN, bool RC>
  static void auto_rc(const M2Args& a, int ckf, int grid, hipStream_t st) {
    switch (ckf) {
      case FMT_F32: m2_auto_kernel<TIN, FMT_F32, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_F16: m2_auto_kernel<TIN, FMT_F16, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_FP8: m2_auto_kernel<TIN, FMT_FP8, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      default: m2_auto_kernel<TIN, FMT_NVFP4, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
    }
  }
  template <typename TIN>
  static void auto_step(const M2Args& a, int ckf, bool rc, int grid, hipStream_t st) {
    if (rc) auto_rc<TIN, true>(a, ckf, grid, st);
    else auto_rc<TIN, false>(a, ckf, grid, st);
  }
  template <typename TIN, int KQ>
  static void spec_append_k(const M2Args& a, int rdf, int grid, hipStream_t st) {
    switch (rdf) {
      case FMT_F32: m2_spec_append_kernel<TIN, FMT_F32, NR, NC, KQ><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_F16: m2_spec_append_kernel<TIN, FMT_F16, NR, NC, KQ><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_FP8: m2_spec_append_kernel<TIN, FMT_FP8, NR, NC, KQ><<<grid, kThreads, 0, st>>>(a); break;
      default: m2_spec_append_kernel<TIN, FMT_NVFP4, NR, NC, KQ><<<grid, kThreads, 0, st>>>(a); break;
    }
  }
  template <typename TIN>
  static void spec_append(const M2Args& a, int rdf, int grid, hipStream_t st) {
    if (a.K <= 1) spec_append_k<TIN, 1>(a, rdf, grid, st);
    else if (a.K <= 2) spec_append_k<TIN, 2>(a, rdf, grid, st);
    else if (a.K <= 4) spec_append_k<TIN, 4>(a, rdf, grid, st);
    else spec_append_k<TIN, 8>(a, rdf, grid, st);
  }
  template <typename TIN, bool RC>
  static void commit_fold_rc(const M2Args& a, int ckf, int grid, hipStream_t st) {
    switch (ckf) {
      case FMT_F32: m2_commit_fold_kernel<TIN, FMT_F32, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_F16: m2_commit_fold_kernel<TIN, FMT_F16, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      case FMT_FP8: m2_commit_fold_kernel<TIN, FMT_FP8, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
      default: m2_commit_fold_kernel<TIN, FMT_NVFP4, RC, NR, NC><<<grid, kThreads, 0, st>>>(a); break;
    }
  }
  template <typename TIN>
  static void commit_fold(const M2Args& a, int ckf, bool rc, int grid, hipStream_t st) {
    if (rc) commit_fold_rc<TIN, true>(a, ckf, grid, st);
    else commit_fold_rc<TIN, false>(a, ckf, grid, st);
  }
  template <typename TIN>
  static void conv_spec(const M2Args& a, int grid, hipStream_t st) {
    m2_conv_spec_kernel<TIN, NR, NC, kMaxDraft><<<grid, kThreads, 0, st>>>(a);
  }
  static void restore(const M2Args& a, int grid, hipStream_t st) {
    m2_restore_kernel<NR, NC><<<grid, kThreads, 0, st>>>(a);
  }
  static void requant(const StateBuf& ck, const StateBuf& rc, int ckf, int grid, hipStream_t st) {
    switch (ckf) {
      case FMT_F32: requant_kernel<FMT_F32, NR, NC><<<grid, kThreads, 0, st>>>(ck, rc); break;
      case FMT_F16: requant_kernel<FMT_F16, NR, NC><<<grid, kThreads, 0, st>>>(ck, rc); break;
      case FMT_FP8: requant_kernel<FMT_FP8, NR, NC><<<grid, kThreads, 0, st>>>(ck, rc); break;
      default: requant_kernel<FMT_NVFP4, NR, NC><<<grid, kThreads, 0, st>>>(ck, rc); break;
    }
  }
};

// Host launcher for one compiled (dstate, headdim) shape; explicitly
// instantiated once per shape in its own translation unit.
template <int NR, int NC>
void m2_launch_shape(M2Op op, const M2Args& a, const M2Launch& l, hipStream_t st) {
  using Sh = M2Shape<NR, NC>;
  const bool bf = l.in_bf16;
  switch (op) {
    case M2Op::Conv:
      if (bf) Sh::template conv<bf16>(a, l.grid, st); else Sh::template conv<float>(a, l.grid, st);
      break;
    case M2Op::NonFlush:
      if (bf) Sh::template nonflush<bf16>(a, l.rdf, l.grid, st); else Sh::template nonflush<float>(a, l.rdf, l.grid, st);
      break;
    case M2Op::Flush:
      if (bf) Sh::template flush<bf16>(a, l.ckf, l.rc, l.grid, st); else Sh::template flush<float>(a, l.ckf, l.rc, l.grid, st);
      break;
    case M2Op::Auto:
      if (bf) Sh::template auto_step<bf16>(a, l.ckf, l.rc, l.grid, st);
      else Sh::template auto_step<float>(a, l.ckf, l.rc, l.grid, st);
      break;
    case M2Op::SpecAppend:
      if (bf) Sh::template spec_append<bf16>(a, l.rdf, l.grid, st); else Sh::template spec_append<float>(a, l.rdf, l.grid, st);
      break;
    case M2Op::CommitFold:
      if (bf) Sh::template commit_fold<bf16>(a, l.ckf, l.rc, l.grid, st); else Sh::template commit_fold<float>(a, l.ckf, l.rc, l.grid, st);
      break;
    case M2Op::ConvSpec:
      if (bf) Sh::template conv_spec<bf16>(a, l.grid, st); else Sh::template conv_spec<float>(a, l.grid, st);
      break;
    case M2Op::Restore:
      Sh::restore(a, l.grid, st);
      break;
    case M2Op::Requant:
      Sh::requant(a.ck, a.rc, l.ckf, l.grid, st);
      break;
  }
}

}  // namespace rs

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
#include "rs_device.h"
#include "rs_tile.h"
#include "rs_internal.h"

namespace rs {

namespace {

// Value columns split across NS workgroups: with k, q, g, beta fixed, column v
// of the stored state (row v of S) evolves and is read out on its own, so a
// workgroup owns the columns c0..c0+NVS-1 of one state and repeats the few
// length-dk dots of the other slices.
template <int NV>
constexpr int gdn_slices() { return NV >= 128 ? 2 : 1; }

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
};

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
        const float al = expf(s.A[e][c]);
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
// U[cur]; returns o[v] = gamma S0 q + ho + kq[cur] u_cur.
template <typename SM>
__device__ __forceinline__ float gdn_finish_row(SM& s, int m, int v, float hu, float ho) {
  const int cur = m - 1;
  const float u = s.bet * (s.vc[v] - s.gam * s.out[0][v]) - hu;
  s.U[cur][v] = u;
  return s.gam * s.out[1][v] + ho + s.kq[cur] * u;
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
    s.W[2][ti] = VG ? expf(gvv) : 0.0f;   // VG: the channel decays
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
template <typename TIN, int NK, int NV, bool VG>
__device__ __forceinline__ void gdn_nonflush_body(const GDNArgs& a, GSmem<NK, NV / gdn_slices<NV>(), VG>& s) {
  constexpr int NVS = NV / gdn_slices<NV>();
  const GPtrs p = gdn_tile<NV, gdn_slices<NV>()>(a);
  rs_meta* mp = a.meta + p.b;
  const int wg = p.h * gdn_slices<NV>() + p.half;
  uint32_t* actr = a.arrive + static_cast<size_t>(p.b) * arrive_groups(a.nv * gdn_slices<NV>()) * kArriveStride;
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
    GSlice<NK, NV, NVS> raw;
    raw.issue(static_cast<const float*>(a.ck.data), p.st, p.c0);
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
    RegTile<4, NK, NVS> S;
    raw.decode(S);
    tile_matvec<2>(S, &s.W[0][0], NK, s.redp(), &s.out[0][0]);
    const int slot = slot_of(nck, len);
    float* ru = static_cast<float*>(a.ru) + (p.st * kRing + slot) * NV + p.c0;
    if (v < NVS) {
      a.o[p.st * NV + p.c0 + v] = gdn_finish_row(s, j, v, hu, ho);
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
  arr.finish(mp, actr, wg, a.nv * gdn_slices<NV>(), MetaOp::NonFlush, 0, nck, len, nd);
}

template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_nonflush_kernel(GDNArgs a) {
  __shared__ GSmem<NK, NV / gdn_slices<NV>(), VG> s;
  gdn_nonflush_body<TIN, NK, NV, VG>(a, s);
}

// ----------------------------------------------------------------------------
// flush step: fold the len held entries and the current token, write once, o
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV, bool VG>
__device__ __forceinline__ void gdn_flush_body(const GDNArgs& a, GSmem<NK, NV / gdn_slices<NV>(), VG>& s) {
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
    GStage<TIN, NK, NV, NVS, VG> stg;
    stg.load(a, p, nck, m);            // records first, then the state tile
    GSlice<NK, NV, NVS> raw;
    raw.issue(ck, p.st, p.c0);
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
    RegTile<4, NK, NVS> S;
    raw.decode(S);
    tile_matvec<2>(S, &s.W[0][0], NK, s.redp(), &s.out[0][0]);
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
    if constexpr (VG) {
      // S0 Diag(gamma_m) + sum_i u_i (r_{m,i} * k_i)^T (k rows decayed above)
      tile_scale_rows(S, s.gv);
      tile_rank_update(S, 1.0f, &s.K[0][0], NK, &s.U[0][0], NVS, m);
    } else {
      tile_rank_update(S, s.gam, &s.K[0][0], NK, &s.U[0][0], NVS, m);
    }
    GSlice<NK, NV, NVS>::store(ck, p.st, p.c0, S);
  }
  arr.finish(mp, actr, wg, a.nv * gdn_slices<NV>(), MetaOp::Flush, 0, nck, len, nd);
}

template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_flush_kernel(GDNArgs a) {
  __shared__ GSmem<NK, NV / gdn_slices<NV>(), VG> s;
  gdn_flush_body<TIN, NK, NV, VG>(a, s);
}

// self-scheduling step (continuous batching): a sequence whose buffer is full
// takes the flush, every other one a non-flush step, in one launch (the branch
// is uniform per workgroup)
template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_auto_kernel(GDNArgs a) {
  __shared__ GSmem<NK, NV / gdn_slices<NV>(), VG> s;
  const GPtrs p = gdn_tile<NV, gdn_slices<NV>()>(a);
  if (a.meta[p.b].len == kRing - 1) gdn_flush_body<TIN, NK, NV, VG>(a, s);
  else gdn_nonflush_body<TIN, NK, NV, VG>(a, s);
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
  float V[KQ][NVS];            // v of the drafts, own columns
  float out[2 * KQ][NVS];      // S0 k_d, S0 q_d
  float kk[KQ][kRing];         // beta_d r_{e,i} (k_e . k_i) for i < e = len + d
  float kq[KQ][kRing];         // r_{e,i} (k_i . q_d) for i <= e
  float rt[KQ][kRing];         // r_{e,i} for i <= e
  float al[kRing];             // alpha of window entry e
  float gam[KQ];               // gamma of draft d's entry (VG: 1, the decays weight the dots)
  float bet[KQ];
  // VG (per-channel decays, e = len + d): WS = k_e * P_d and q_d * P_d with
  // P_d = prod_{len<=l<=e} alpha_l; DW[d(d-1)/2 + j] = prod_{len+j<l<=e} alpha_l
  // (the decay between draft j and draft d > j)
  alignas(16) float WS[VG ? 2 * KQ : 1][NK];
  alignas(16) float DW[VG && KQ > 1 ? KQ * (KQ - 1) / 2 : 1][NK];
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
template <int Q, int NK, int NVS>
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

}  // namespace

// Without the per-channel gate and up to 4 drafts: 7 waves per SIMD with the
// matrix-core accumulators, the register budget the VALU dots and matvecs had;
// otherwise the compiler puts the accumulators in separate registers and
// occupancy drops.
template <typename TIN, int NK, int NV, int KQ, bool VG>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu((!VG && KQ <= 4) ? 7 : 1, 8)))
void gdn_spec_append_kernel(GDNArgs a) {
  constexpr int NS = gdn_slices<NV>();
  constexpr int NVS = NV / NS;
  constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  static_assert(NK % VK == 0 && NVS % VK == 0, "records are whole 16-byte chunks");
  constexpr int CK = (kRing * NK / VK + kThreads - 1) / kThreads;
  constexpr int CU = (kRing * NVS / 4 + kThreads - 1) / kThreads;
  constexpr int CD = (KQ * NK / VK + kThreads - 1) / kThreads;
  constexpr int CV = (KQ * NVS / VK + kThreads - 1) / kThreads;
  __shared__ GSpecSmem<NK, NVS, KQ, VG> s;
  const GPtrs p = gdn_tile<NV, NS>(a);
  const int K = a.K;
  static_assert(!VG || NK <= kThreads, "one thread per key channel");
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
    RegChunks<TIN, CD> cq, cd;
    RegChunks<TIN, CV> cv;
    ck.load(EntrySrc<TIN>{rk, ik, kstride, nck, len, NK}, n, NK);
    cu.load(EntrySrc<float>{ru, ru, 0, nck, len, NV}, len, NVS);
    cq.load(EntrySrc<TIN>{iq, iq, kstride, 0, 0, NK}, K, NK);
    cd.load(EntrySrc<TIN>{ik, ik, kstride, 0, 0, NK}, K, NK);
    cv.load(EntrySrc<TIN>{iv, iv, vstride, 0, 0, NVS}, K, NVS);
    float gv = 0.0f;
    float lg[kRing];   // VG: the log decays of window entries 0..n-1 of this thread's key channel
    if constexpr (VG) {
      const int c = static_cast<int>(threadIdx.x) < NK ? static_cast<int>(threadIdx.x) : NK - 1;
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
    GSlice<NK, NV, NVS> raw;
    raw.issue(static_cast<const float*>(a.ck.data), p.st, p.c0);
    arr.arrive(actr, wg, nck, len, nd);
    ck.to_lds(&s.K[0][0], NK, n, NK);
    cu.to_lds(&s.U[0][0], NVS, len, NVS);
    cd.to_lds(&s.W[0][0], 2 * NK, K, NK);
    cq.to_lds(&s.W[1][0], 2 * NK, K, NK);
    for (int idx = 2 * K * NK + threadIdx.x; idx < 2 * KQ * NK; idx += kThreads) (&s.W[0][0])[idx] = 0.0f;
    cv.to_lds(&s.V[0][0], NVS, K, NVS);
    if constexpr (!VG)
      if (static_cast<int>(threadIdx.x) < n) s.al[threadIdx.x] = expf(gv);
    if (static_cast<int>(threadIdx.x) < K) s.bet[threadIdx.x] = bv;
    __syncthreads();
    if constexpr (VG) {
      // The decay from entry i to draft entry e = len + d factors at the first
      // draft: r_{e,i} = Rh_i * P_d for a held entry (Rh_i = prod_{i<l<len}
      // alpha_l), and DW for a pair of drafts. Channel owners (one thread per
      // key channel, window decays in registers) scale the held k rows by Rh in
      // place and write WS and DW; then every dot of every draft in one pass:
      //   kk[d][i] = beta_d <k_e, r_{e,i} * k_i>,  kq[d][i] = <q_d, r_{e,i} * k_i>.
      // gamma_e = Gam * P_d with Gam = prod_{l<len} alpha_l.
      const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
      float gam_c = 1.0f;
      if (static_cast<int>(threadIdx.x) < NK) {
        const int c = threadIdx.x;
#pragma unroll
        for (int e = 0; e < kRing; ++e) lg[e] = expf(lg[e]);   // alpha per entry
        float acc = 1.0f;
#pragma unroll
        for (int i = kRing - 1; i >= 0; --i) {
          if (i < len) {
            s.K[i][c] *= acc;
            acc *= lg[i];
          }
        }
        gam_c = acc;
        float pd = 1.0f;
        for (int d = 0; d < K; ++d) {
          pd *= lg[len + d];                      // len + d < 16; wave-uniform index
          s.WS[2 * d][c] = s.W[2 * d][c] * pd;
          s.WS[2 * d + 1][c] = s.W[2 * d + 1][c] * pd;
          float q = 1.0f;
          for (int j = d - 1; j >= 0; --j) {
            q *= lg[len + j + 1];
            s.DW[d * (d - 1) / 2 + j][c] = q;
          }
        }
      }
      if (static_cast<int>(threadIdx.x) < K) s.gam[threadIdx.x] = 1.0f;
      __syncthreads();
      // pairs of draft d: len held kk, len held kq, d draft kk, d + 1 draft kq
      const int npairs = K * (2 * len + 1) + K * (K - 1);
      for (int pr = grp; pr < npairs; pr += kThreads / 16) {
        int d = 0, r = pr;
        while (r >= 2 * (len + d) + 1) {          // uniform over the group
          r -= 2 * (len + d) + 1;
          ++d;
        }
        const int ee = len + d;
        float part;
        bool isq;
        int i;
        if (r < 2 * len) {                        // held entry i: k row already scaled by Rh_i
          isq = r >= len;
          i = isq ? r - len : r;
          part = lds_dot16<NK>(&s.K[i][0], &s.WS[2 * d + (isq ? 1 : 0)][0], ln);
        } else {                                  // earlier draft j (kk: j < d; kq: j <= d)
          const int t = r - 2 * len;
          isq = t >= d;
          const int j = isq ? t - d : t;
          i = len + j;
          const float* w = j < d ? &s.DW[d * (d - 1) / 2 + j][0] : nullptr;
          part = lds_dot16<NK>(&s.K[i][0], isq ? &s.W[2 * d + 1][0] : &s.K[ee][0], ln, w);
        }
        part = group_sum16(part);
        if (ln == 0) {
          if (isq) s.kq[d][i] = part;
          else s.kk[d][i] = s.bet[d] * part;
        }
      }
      __syncthreads();
      // matvec weights gamma_e * k_e and gamma_e * q_d (owners: their channel)
      if (static_cast<int>(threadIdx.x) < NK) {
        for (int d = 0; d < K; ++d) {
          s.W[2 * d][threadIdx.x] = s.WS[2 * d][threadIdx.x] * gam_c;
          s.W[2 * d + 1][threadIdx.x] = s.WS[2 * d + 1][threadIdx.x] * gam_c;
        }
      }
    } else {
      // decays r_{e,i} (direct products), one (draft, entry) pair per thread, and gamma
      for (int idx = threadIdx.x; idx < K * kRing; idx += kThreads) {
        const int d = idx / kRing, i = idx - d * kRing, ee = len + d;
        if (i <= ee) {
          float r = 1.0f;
          for (int l = i + 1; l <= ee; ++l) r *= s.al[l];
          s.rt[d][i] = r;
          if (i == 0) s.gam[d] = r * s.al[0];
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
    RegTile<4, NK, NVS> S;
    raw.decode(S);
    // S0 [k_d, q_d]: all 2 KQ weight rows in one pass on the matrix cores where the
    // slice has 64 columns and the scratch holds it (without the per-channel gate:
    // with it the accumulators cost a wave of occupancy); otherwise on the VALU, rows
    // 0..KQ-1, then KQ..2KQ-1 if drafts reach them (fewer accumulator registers and
    // half the scratch of one 2KQ-row pass). Barriers inside publish the dots.
    constexpr bool kMfmaMv = !VG && NVS == 64 && 4 * 2 * KQ * NVS <= GSpecSmem<NK, NVS, KQ, VG>::KROWS * NK;
    if constexpr (kMfmaMv) {
      tile_matvec_mfma<2 * KQ>(S, &s.W[0][0], NK, red, &s.out[0][0]);
    } else {
      tile_matvec<KQ>(S, &s.W[0][0], NK, red, &s.out[0][0]);
      if (2 * K > KQ) tile_matvec<KQ>(S, &s.W[KQ][0], NK, red, &s.out[KQ][0]);
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
      HU[d * NVS + v] = s.bet[d] * (s.V[d][v] - s.gam[d] * s.out[2 * d][v]) - hu;
      HO[d * NVS + v] = s.gam[d] * s.out[2 * d + 1][v] + ho;
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
    // drafts into the ring (bit copies); each slice its own v columns
    TIN* rv = static_cast<TIN*>(a.rv) + p.st * kRing * NV + p.c0;
    const auto dslot = [&](int d) { return slot_of(nck, len + d); };
    copy_rows16(rv, NV, iv, vstride, K, NVS, dslot);
    if (p.half == 0) {
      if (static_cast<int>(threadIdx.x) < K) {
        const int d = threadIdx.x, sl = slot_of(nck, len + d);
        if constexpr (!VG) static_cast<float*>(a.rg)[p.st * kRing + sl] = a.g[d * gstride + p.st];
        static_cast<float*>(a.rbeta)[p.st * kRing + sl] = a.beta[d * gstride + p.st];
      }
      if constexpr (VG) {
        float* rgw = static_cast<float*>(a.rg) + p.st * kRing * NK;
        copy_rows16(rgw, NK, a.g + p.st * NK, gstride * NK, K, NK, dslot);
      }
      if (p.h % a.vpk == 0) {
        TIN* rkw = static_cast<TIN*>(a.rk) + bk * kRing * NK;
        TIN* rqw = static_cast<TIN*>(a.rq) + bk * kRing * NK;
        copy_rows16(rkw, NK, ik, kstride, K, NK, dslot);
        copy_rows16(rqw, NK, iq, kstride, K, NK, dslot);
      }
    }
  }
  arr.finish(mp, actr, wg, a.nv * NS, MetaOp::Append, K, nck, len, nd);
}

// ----------------------------------------------------------------------------
// speculative commit (ReplaySSM), fold part: for each sequence listed by
// commit_meta, S <- gamma_m S0 + sum_i r_{m,i} u_i k_i^T over its m committed
// entries (u rows from the ring), one column slice per work item, over a
// fixed grid (every workgroup leaves when the list is done). VG (KDA):
// S <- S0 Diag(gamma_m) + sum_i u_i (r_{m,i} * k_i)^T with per-channel decays.
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV, bool VG>
__global__ __launch_bounds__(kThreads) void gdn_commit_fold_kernel(GDNArgs a) {
  constexpr int NS = gdn_slices<NV>();
  constexpr int NVS = NV / NS;
  constexpr int VK = 16 / static_cast<int>(sizeof(TIN));
  constexpr int CK = (kRing * NK / VK + kThreads - 1) / kThreads;
  constexpr int CU = (kRing * NVS / 4 + kThreads - 1) / kThreads;
  static_assert(!VG || NK <= kThreads, "one thread per key channel");
  __shared__ GSmem<NK, NVS, VG> s;
  const int per = a.nv * NS;
  const int total = *a.work_count * per;
  float* ckp = static_cast<float*>(a.ck.data);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const FoldItem it = a.work[item / per];
    const int r = item - (item / per) * per;
    const int h = r / NS, half = r - h * NS, c0 = half * NVS, m = it.m;
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
    GSlice<NK, NV, NVS> raw;
    raw.issue(ckp, st, c0);
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
            acc *= expf(lg[i]);
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
    RegTile<4, NK, NVS> S;
    raw.decode(S);
    if constexpr (VG) {
      tile_scale_rows(S, s.gv);
      tile_rank_update(S, 1.0f, &s.K[0][0], NK, &s.U[0][0], NVS, m);
    } else {
      tile_rank_update(S, s.gam, &s.K[0][0], NK, &s.U[0][0], NVS, m);
    }
    GSlice<NK, NV, NVS>::store(ckp, st, c0, S);
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
    for (int idx = threadIdx.x; idx < K * NK; idx += kThreads) (&s.AL[0][0])[idx] = expf((&s.AL[0][0])[idx]);
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

template <int NK, int NV, bool VG>
struct gdn_step_kernels {
  static void conv(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if (bf) gdn_conv_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_conv_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  }
  static void nonflush(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if (bf) gdn_nonflush_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_nonflush_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  }
  static void flush(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if (bf) gdn_flush_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_flush_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  }
  static void auto_step(bool bf, const GDNArgs& a, int grid, hipStream_t st) {
    if (bf) gdn_auto_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_auto_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  }
};

template <typename TIN, int NK, int NV, bool VG>
void gdn_spec_append(const GDNArgs& a, int grid, hipStream_t st) {
  if (a.K <= 2) gdn_spec_append_kernel<TIN, NK, NV, 2, VG><<<grid, kThreads, 0, st>>>(a);
  else if (a.K <= 4) gdn_spec_append_kernel<TIN, NK, NV, 4, VG><<<grid, kThreads, 0, st>>>(a);
  else gdn_spec_append_kernel<TIN, NK, NV, 8, VG><<<grid, kThreads, 0, st>>>(a);
}

template <typename TIN, int NK, int NV, bool VG>
void gdn_conv_spec(const GDNArgs& a, int grid, hipStream_t st) {
  if (a.K <= 2) gdn_conv_spec_kernel<TIN, NK, NV, 2, VG><<<grid, kThreads, 0, st>>>(a);
  else if (a.K <= 4) gdn_conv_spec_kernel<TIN, NK, NV, 4, VG><<<grid, kThreads, 0, st>>>(a);
  else gdn_conv_spec_kernel<TIN, NK, NV, 8, VG><<<grid, kThreads, 0, st>>>(a);
}

template <int NK, int NV, bool VG>
void gdn_spec_kernels(GDNOp op, bool bf, const GDNArgs& a, int grid, hipStream_t st) {
  if (op == GDNOp::SpecAppend) {
    if (bf) gdn_spec_append<bf16, NK, NV, VG>(a, grid, st);
    else gdn_spec_append<float, NK, NV, VG>(a, grid, st);
  } else if (op == GDNOp::ConvSpec) {
    if (bf) gdn_conv_spec<bf16, NK, NV, VG>(a, grid, st);
    else gdn_conv_spec<float, NK, NV, VG>(a, grid, st);
  } else {
    if (bf) gdn_commit_fold_kernel<bf16, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
    else gdn_commit_fold_kernel<float, NK, NV, VG><<<grid, kThreads, 0, st>>>(a);
  }
}

template <int NK, int NV>
void gdn_launch_shape(GDNOp op, const GDNArgs& a, GDNLaunch l, hipStream_t st) {
  const bool bf = l.in_bf16;
  // replay steps and appends: one workgroup per column slice of each state
  if (op == GDNOp::NonFlush || op == GDNOp::Flush || op == GDNOp::Auto || op == GDNOp::SpecAppend ||
      op == GDNOp::ConvSpec)
    l.grid *= gdn_slices<NV>();
  switch (op) {
    case GDNOp::Conv:
      if (l.vg) gdn_step_kernels<NK, NV, true>::conv(bf, a, l.grid, st);
      else gdn_step_kernels<NK, NV, false>::conv(bf, a, l.grid, st);
      break;
    case GDNOp::NonFlush:
      if (l.vg) gdn_step_kernels<NK, NV, true>::nonflush(bf, a, l.grid, st);
      else gdn_step_kernels<NK, NV, false>::nonflush(bf, a, l.grid, st);
      break;
    case GDNOp::Flush:
      if (l.vg) gdn_step_kernels<NK, NV, true>::flush(bf, a, l.grid, st);
      else gdn_step_kernels<NK, NV, false>::flush(bf, a, l.grid, st);
      break;
    case GDNOp::Auto:
      if (l.vg) gdn_step_kernels<NK, NV, true>::auto_step(bf, a, l.grid, st);
      else gdn_step_kernels<NK, NV, false>::auto_step(bf, a, l.grid, st);
      break;
    case GDNOp::SpecAppend:
    case GDNOp::ConvSpec:
      if (l.vg) gdn_spec_kernels<NK, NV, true>(op, bf, a, l.grid, st);
      else gdn_spec_kernels<NK, NV, false>(op, bf, a, l.grid, st);
      break;
    case GDNOp::CommitFold: {
      const int items = l.grid * gdn_slices<NV>();   // upper bound of listed work items
      const int grid = items < 2048 ? items : 2048;
      if (l.vg) gdn_spec_kernels<NK, NV, true>(op, bf, a, grid, st);
      else gdn_spec_kernels<NK, NV, false>(op, bf, a, grid, st);
      break;
    }
    case GDNOp::Restore:
      gdn_restore_kernel<NK, NV><<<l.grid, kThreads, 0, st>>>(a);
      break;
  }
}

}  // namespace

bool gdn_shape_supported(int dk, int dv) {
  return (dk == 16 && dv == 16) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128);
}

void gdn_launch(GDNOp op, const GDNArgs& a, const GDNLaunch& l, hipStream_t st) {
  if (l.dk == 16 && l.dv == 16) gdn_launch_shape<16, 16>(op, a, l, st);
  else if (l.dk == 64 && l.dv == 64) gdn_launch_shape<64, 64>(op, a, l, st);
  else if (l.dk == 128 && l.dv == 128) gdn_launch_shape<128, 128>(op, a, l, st);
}

}  // namespace rs

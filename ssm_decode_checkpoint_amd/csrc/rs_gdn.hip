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
// One 256-thread workgroup per (sequence, value head) state, stored as
// [dk][dv] (value index innermost) so that S0 k and S0 q are sums over rows
// held in registers. The j+1 matrix-vector products S0 [k_1 .. k_j, q_j]
// share the single read of S0; the triangular solve (size <= 16) and the
// output combination run on LDS vectors of length dv.
#include "rs_device.h"
#include "rs_tile.h"
#include "rs_internal.h"

namespace rs {

namespace {

template <int NK, int NV>
struct GSmem {
  float W[kRing + 4][NK];    // k_1 .. k_m, then q, then zero rows up to the matvec chunk
  float V[kRing][NV];        // v_i; reused for the fold columns r_{m,i} u_i
  float U[kRing][NV];        // u_i
  float out[kRing + 4][NV];  // S0 W_r
  float red[4 * 4 * NV];
  float KK[kRing][kRing];    // beta_i r_{i,l} (k_i . k_l), l < i
  float coef[kRing];         // r_{j,i} (k_i . q_j)
  float al[kRing], be[kRing], gam[kRing];
  float s4[4];
};

template <typename TIN>
__device__ __forceinline__ const TIN* ring_row(const TIN* base, long long nck, int e, int width) {
  return base + static_cast<size_t>((nck + e) & (kRing - 1)) * width;
}

// Load n records (entries 0..n-1: ring for e < nring, `cur` for e == nring) into LDS rows.
template <typename TIN>
__device__ __forceinline__ void stage(float* dst, int stride, const TIN* ring, const TIN* cur, long long nck,
                                      int nring, int n, int width) {
  for (int idx = threadIdx.x; idx < n * width; idx += kThreads) {
    const int e = idx / width, r = idx - e * width;
    const TIN* src = e < nring ? ring_row(ring, nck, e, width) : cur;
    dst[e * stride + r] = to_f(src[r]);
  }
}

struct GPtrs {
  size_t tile;
  int b, h, kh;
};

__device__ __forceinline__ GPtrs gdn_tile(const GDNArgs& a) {
  GPtrs p;
  p.tile = static_cast<size_t>(xcd_tile(blockIdx.x, gridDim.x));
  p.b = static_cast<int>(p.tile / a.nv);
  p.h = static_cast<int>(p.tile - static_cast<size_t>(p.b) * a.nv);
  p.kh = p.h / a.vpk;
  return p;
}

// Stage entries 0..m-1 (k into W rows, v into V rows, alpha, beta), with the
// current token as entry m-1 when cur is true, and the read vector q into W[m].
template <typename TIN, int NK, int NV>
__device__ __forceinline__ void gdn_stage(GSmem<NK, NV>& s, const GDNArgs& a, const GPtrs& p, long long nck,
                                          int nring, int m, bool with_q) {
  const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
  const TIN* rk = static_cast<const TIN*>(a.rk) + bk * kRing * NK;
  const TIN* rv = static_cast<const TIN*>(a.rv) + p.tile * kRing * NV;
  const float* rg = static_cast<const float*>(a.rg) + p.tile * kRing;
  const float* rbt = static_cast<const float*>(a.rbeta) + p.tile * kRing;
  const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
  const TIN* iv = static_cast<const TIN*>(a.v) + p.tile * NV;
  stage(&s.W[0][0], NK, rk, ik, nck, nring, m, NK);
  stage(&s.V[0][0], NV, rv, iv, nck, nring, m, NV);
  if (with_q) {
    const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
    for (int i = threadIdx.x; i < NK; i += kThreads) s.W[m][i] = to_f(iq[i]);
  }
  // zero the rows after the staged ones that a 4-wide matvec chunk may read
  // (up to the end of the chunk holding the last row, and the 4 rows from q)
  const int used = m + (with_q ? 1 : 0);
  int end = (used + 3) & ~3;
  if (with_q && end < m + 4) end = m + 4;
  for (int idx = used * NK + threadIdx.x; idx < end * NK; idx += kThreads) (&s.W[0][0])[idx] = 0.0f;
  if (static_cast<int>(threadIdx.x) < m) {
    const int e = threadIdx.x;
    const bool ring = e < nring;
    const float g = ring ? rg[(nck + e) & (kRing - 1)] : a.g[p.tile];
    const float bt = ring ? rbt[(nck + e) & (kRing - 1)] : a.beta[p.tile];
    s.al[e] = expf(g);
    s.be[e] = bt;
  }
}

// S0 W_r for rows r < rows (in chunks of four weight vectors); results in s.out.
template <int NK, int NV>
__device__ __forceinline__ void gdn_products(const RegTile<4, NK, NV>& S, GSmem<NK, NV>& s, int rows) {
  for (int q0 = 0; q0 < rows; q0 += 4) tile_matvec<4>(S, &s.W[q0][0], NK, s.red, &s.out[q0][0]);
}

// r_{t,i} = prod_{i<l<=t} alpha_l (0-based entries)
__device__ __forceinline__ float decay_between(const float* al, int i, int t) {
  float r = 1.0f;
  for (int l = i + 1; l <= t; ++l) r *= al[l];
  return r;
}

// Gram terms, gammas, then u_0..u_{m-1} by forward substitution (u in s.U).
// If with_q, also coef[i] = r_{m-1,i} (k_i . q) for the output.
template <int NK, int NV>
__device__ __forceinline__ void gdn_solve(GSmem<NK, NV>& s, int m, bool with_q) {
  const int grp = threadIdx.x >> 4, ln = threadIdx.x & 15;
  // pairs (i, l) with l < i < m, plus (i, q) for i < m when with_q
  const int npair = m * (m - 1) / 2;
  const int ntot = npair + (with_q ? m : 0);
  for (int pr = grp; pr < ntot; pr += kThreads / 16) {
    int i, l;
    if (pr < npair) {
      i = 1;
      int rem = pr;
      while (rem >= i) { rem -= i; ++i; }
      l = rem;
    } else {
      i = pr - npair;
      l = m;  // the q row
    }
    float part = 0.0f;
    for (int n = ln; n < NK; n += 16) part += s.W[i][n] * s.W[l][n];
    part = group_sum16(part);
    if (ln == 0) {
      if (l < m) s.KK[i][l] = s.be[i] * decay_between(s.al, l, i) * part;
      else s.coef[i] = decay_between(s.al, i, m - 1) * part;
    }
  }
  if (threadIdx.x == 0) {
    float gm = 1.0f;
    for (int e = 0; e < m; ++e) {
      gm *= s.al[e];
      s.gam[e] = gm;
    }
  }
  __syncthreads();
  for (int v = threadIdx.x; v < NV; v += kThreads) {
    for (int i = 0; i < m; ++i) {
      float u = s.be[i] * (s.V[i][v] - s.gam[i] * s.out[i][v]);
      for (int l = 0; l < i; ++l) u -= s.KK[i][l] * s.U[l][v];
      s.U[i][v] = u;
    }
  }
  __syncthreads();
}

}  // namespace

// ----------------------------------------------------------------------------
// conventional step (baseline)
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV>
__global__ __launch_bounds__(kThreads) void gdn_conv_kernel(GDNArgs a) {
  __shared__ GSmem<NK, NV> s;
  const GPtrs p = gdn_tile(a);
  RawTile<FMT_F32, 4, NK, NV> raw;
  raw.issue(a.ck, p.tile);
  const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
  const TIN* ik = static_cast<const TIN*>(a.k) + bk * NK;
  const TIN* iq = static_cast<const TIN*>(a.q) + bk * NK;
  const TIN* iv = static_cast<const TIN*>(a.v) + p.tile * NV;
  for (int i = threadIdx.x; i < NK; i += kThreads) {
    s.W[0][i] = to_f(ik[i]);
    s.W[1][i] = to_f(iq[i]);
    s.W[2][i] = 0.0f;
    s.W[3][i] = 0.0f;
  }
  for (int i = threadIdx.x; i < NV; i += kThreads) s.V[0][i] = to_f(iv[i]);
  __syncthreads();
  // k . q (one 16-lane group)
  if (threadIdx.x < 16) {
    float part = 0.0f;
    for (int n = threadIdx.x; n < NK; n += 16) part += s.W[0][n] * s.W[1][n];
    part = group_sum16(part);
    if (threadIdx.x == 0) s.coef[0] = part;
  }
  const float alpha = expf(a.g[p.tile]);
  const float beta = a.beta[p.tile];
  RegTile<4, NK, NV> S;
  raw.decode(S);
  tile_matvec<4>(S, &s.W[0][0], NK, s.red, &s.out[0][0]);   // out[0] = S k, out[1] = S q
  for (int v = threadIdx.x; v < NV; v += kThreads) s.U[0][v] = beta * (s.V[0][v] - alpha * s.out[0][v]);
  __syncthreads();
  tile_rank_update(S, alpha, &s.W[0][0], NK, &s.U[0][0], NV, 1);
  tile_store<FMT_F32>(a.ck, p.tile, S, s.s4);
  const float kq = s.coef[0];
  for (int v = threadIdx.x; v < NV; v += kThreads) a.o[p.tile * NV + v] = alpha * s.out[1][v] + kq * s.U[0][v];
}

// ----------------------------------------------------------------------------
// non-flush step: o from checkpoint + buffer (UT form), append, no state write
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV>
__global__ __launch_bounds__(kThreads) void gdn_nonflush_kernel(GDNArgs a) {
  __shared__ GSmem<NK, NV> s;
  const GPtrs p = gdn_tile(a);
  rs_meta* mp = a.meta + p.b;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 2 ? RS_ERR_FULL : 0);
  if (errbit == 0) {
    const int j = len + 1;
    RawTile<FMT_F32, 4, NK, NV> raw;
    raw.issue(a.ck, p.tile);
    gdn_stage<TIN>(s, a, p, nck, len, j, true);
    __syncthreads();
    RegTile<4, NK, NV> S;
    raw.decode(S);
    gdn_products(S, s, j + 1);                 // barriers inside publish the staged rows too
    gdn_solve(s, j, true);
    const float gj = s.gam[j - 1];
    for (int v = threadIdx.x; v < NV; v += kThreads) {
      float o = gj * s.out[j][v];
      for (int i = 0; i < j; ++i) o += s.coef[i] * s.U[i][v];
      a.o[p.tile * NV + v] = o;
    }
    // append the current record (bit copies)
    const int slot = static_cast<int>((nck + len) & (kRing - 1));
    const size_t bk = static_cast<size_t>(p.b) * a.nqk + p.kh;
    TIN* rv = static_cast<TIN*>(a.rv) + p.tile * kRing * NV;
    const TIN* iv = static_cast<const TIN*>(a.v) + p.tile * NV;
    for (int v = threadIdx.x; v < NV; v += kThreads) rv[slot * NV + v] = iv[v];
    if (threadIdx.x == 0) {
      static_cast<float*>(a.rg)[p.tile * kRing + slot] = a.g[p.tile];
      static_cast<float*>(a.rbeta)[p.tile * kRing + slot] = a.beta[p.tile];
    }
    if (p.h % a.vpk == 0) {
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
  arrive_and_update(mp, a.nv, [&](rs_meta* m) {
    if (errbit) m->err |= errbit;
    else m->len = len + 1;
  });
}

// ----------------------------------------------------------------------------
// flush step: fold the len stored entries and the current token, write once, o
// ----------------------------------------------------------------------------
template <typename TIN, int NK, int NV>
__global__ __launch_bounds__(kThreads) void gdn_flush_kernel(GDNArgs a) {
  __shared__ GSmem<NK, NV> s;
  const GPtrs p = gdn_tile(a);
  rs_meta* mp = a.meta + p.b;
  const int len = mp->len, nd = mp->nd;
  const long long nck = mp->n_ckpt;
  const int errbit = nd != 0 ? RS_ERR_PENDING : (len > kRing - 1 ? RS_ERR_FULL : 0);
  const int m = len + 1;
  if (errbit == 0) {
    RawTile<FMT_F32, 4, NK, NV> raw;
    raw.issue(a.ck, p.tile);
    gdn_stage<TIN>(s, a, p, nck, len, m, true);
    __syncthreads();
    RegTile<4, NK, NV> S;
    raw.decode(S);
    gdn_products(S, s, m);
    gdn_solve(s, m, false);
    // fold columns r_{m,i} u_i into V (v is no longer needed)
    for (int idx = threadIdx.x; idx < m * NV; idx += kThreads) {
      const int i = idx / NV, v = idx - i * NV;
      s.V[i][v] = decay_between(s.al, i, m - 1) * s.U[i][v];
    }
    __syncthreads();
    tile_rank_update(S, s.gam[m - 1], &s.W[0][0], NK, &s.V[0][0], NV, m);
    // o = S_m q from the folded state (q sits in W[m]; W[m+1..] are zero)
    tile_matvec<4>(S, &s.W[m][0], NK, s.red, &s.out[0][0]);
    for (int v = threadIdx.x; v < NV; v += kThreads) a.o[p.tile * NV + v] = s.out[0][v];
    tile_store<FMT_F32>(a.ck, p.tile, S, s.s4);
  }
  arrive_and_update(mp, a.nv, [&](rs_meta* mm) {
    if (errbit) {
      mm->err |= errbit;
    } else {
      mm->n_ckpt = nck + m;
      mm->len = 0;
    }
  });
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
namespace {

template <int NK, int NV>
void gdn_launch_shape(GDNOp op, const GDNArgs& a, const GDNLaunch& l, hipStream_t st) {
  const bool bf = l.in_bf16;
  switch (op) {
    case GDNOp::Conv:
      if (bf) gdn_conv_kernel<bf16, NK, NV><<<l.grid, kThreads, 0, st>>>(a);
      else gdn_conv_kernel<float, NK, NV><<<l.grid, kThreads, 0, st>>>(a);
      break;
    case GDNOp::NonFlush:
      if (bf) gdn_nonflush_kernel<bf16, NK, NV><<<l.grid, kThreads, 0, st>>>(a);
      else gdn_nonflush_kernel<float, NK, NV><<<l.grid, kThreads, 0, st>>>(a);
      break;
    case GDNOp::Flush:
      if (bf) gdn_flush_kernel<bf16, NK, NV><<<l.grid, kThreads, 0, st>>>(a);
      else gdn_flush_kernel<float, NK, NV><<<l.grid, kThreads, 0, st>>>(a);
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

// gfx950 kernels of the on-device SVD of a delta ("Delta-CoMe - 清华联合
// OpenBMB...", technical principles: low-rank decomposition of the delta;
// "Enhancing Delta Compression in LLMs via SVD-based Quantization Error
// Minimization", §2.4 step 1: the SVD of ΔW before the bit allocation and
// quantization): the r leading singular pairs of A = delta [out][in], fp32,
// in the host packer's layout (U [r][out], sigma [r], V [r][in]).
//
// With m = min(out, in): G = A^T A (in <= out) or A A^T (out < in), m x m,
// accumulated in fp64 from the fp32 entries (every product exact).  G's
// eigenpairs (lambda_i = sigma_i^2 and the right, resp. left, singular
// vectors) come from block Jacobi: G is cut into 32-index blocks, padded to
// an even count; a sweep runs every pair of blocks once in a round-robin
// tournament (rounds of disjoint pairs, in parallel).  A pair's 64 x 64
// principal submatrix S is diagonalized in LDS by cyclic Jacobi (rounds of
// 32 disjoint plane rotations, each zeroing S_ab: the stable symmetric Schur
// rotation), giving Q with Q^T S Q diagonal; then G <- Q^T G Q on the pair's
// rows and columns and the eigenvector rows W <- Q^T W.  Sweeps stop when
// every pair of a sweep met its submatrix already diagonal:
// |S_ab| <= 1e-13 (sqrt(|S_aa S_bb|) + trace(G) / 10).  The other vectors
// follow as A v / sigma (resp. A^T u / sigma) in fp64 sums; each pair is
// signed so that the largest-magnitude entry of v is positive (lowest index
// on ties).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "dc_internal.h"

namespace dc {
namespace {

constexpr int kSB = 32;        // indices per Jacobi block
constexpr int kSP = 2 * kSB;   // indices of a pair's submatrix
constexpr int kST = 64;        // tile edge of the Gram and output products
constexpr int kSK = 32;        // K chunk of those products

// Players a < b of match `idx` in round `k` of a round-robin tournament of
// n (even) players: player n - 1 stays, the others rotate.
__device__ __forceinline__ void pair_of(int n, int k, int idx, int& a, int& b) {
  int x, y;
  if (idx == 0) {
    x = n - 1;
    y = k;
  } else {
    x = (k + idx) % (n - 1);
    y = (k - idx + (n - 1)) % (n - 1);
  }
  a = min(x, y);
  b = max(x, y);
}

// Global index of local index e (< kSP) of the pair of blocks (I, J).
__device__ __forceinline__ int gidx(int I, int J, int e) { return e < kSB ? I * kSB + e : J * kSB + (e - kSB); }

// G = A'^T A' over the n rows of A' (m x m, padded to mp, fp64): A' = A
// [n][m] when !trans, A' = A^T when trans (A [m][n]).  Block: a 64 x 64 tile
// (ti <= tj; the mirror tile is written too), 4 x 4 outputs per thread.
// Also sets flag to 1 if an entry of A is not finite.
__global__ void __launch_bounds__(256) k_gram(const float* __restrict__ A, int m, int n, int trans, int mp,
                                              double* __restrict__ G, uint32_t* __restrict__ flag) {
  const int ti = blockIdx.x, tj = blockIdx.y;
  if (tj < ti) return;
  __shared__ float As[kSK][kST + 1], Bs[kSK][kST + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int i0 = ti * kST, j0 = tj * kST;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  bool bad = false;
  // element (k, c) of A'^T ... : A'[k][c] (k < n rows of A', c < m columns)
  auto at = [&](int k, int c) -> float {
    if (k >= n || c >= m) return 0.f;
    return trans ? A[(size_t)c * n + k] : A[(size_t)k * m + c];
  };
  for (int k0 = 0; k0 < n; k0 += kSK) {
    for (int e = tid; e < kSK * kST; e += 256) {
      // !trans: consecutive threads along the columns (a row of A); trans: along k
      const int kk = trans ? (e % kSK) : (e / kST), cc = trans ? (e / kSK) : (e % kST);
      const float va = at(k0 + kk, i0 + cc), vb = at(k0 + kk, j0 + cc);
      bad = bad || !isfinite(va) || !isfinite(vb);
      As[kk][cc] = va;
      Bs[kk][cc] = vb;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kSK; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = (double)As[k][4 * ty + u];
        b[u] = (double)Bs[k][4 * tx + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  if (bad) *flag = 1u;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + 4 * ty + u, j = j0 + 4 * tx + v;   // < mp: mp is a multiple of kST
      G[(size_t)i * mp + j] = acc[u][v];
      G[(size_t)j * mp + i] = acc[u][v];
    }
}

// W = I (mp x mp), the convergence words zeroed.
__global__ void __launch_bounds__(256) k_eye(double* __restrict__ W, int mp, unsigned long long* __restrict__ off,
                                             int noff) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (size_t)noff) off[i] = 0ull;
  if (i >= (size_t)mp * mp) return;
  W[i] = (i / mp == i % mp) ? 1.0 : 0.0;
}

// One pair of blocks of round `round`: S = G[P][P] for P = I u J, its
// relative off-diagonal size (before) into off (max, as bits of a
// non-negative double), then cyclic Jacobi on S until it is diagonal to
// the working precision; Q (S <- Q^T S Q) goes to Qall[pair].
__global__ void __launch_bounds__(256) k_bj_eig(const double* __restrict__ G, int mp, int nb, int round,
                                                double floor_abs, double* __restrict__ Qall,
                                                unsigned long long* __restrict__ off) {
  __shared__ double S[kSP][kSP + 1], Q[kSP][kSP + 1];
  __shared__ double cs[kSP / 2], sn[kSP / 2];
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int I, J;
  pair_of(nb, round, blockIdx.x, I, J);
  for (int e = tid; e < kSP * kSP; e += 256) {
    const int a = e / kSP, b = e % kSP;
    S[a][b] = G[(size_t)gidx(I, J, a) * mp + gidx(I, J, b)];
    Q[a][b] = a == b ? 1.0 : 0.0;
  }
  __syncthreads();
  // largest |S_ab| / (sqrt(|S_aa S_bb|) + floor_abs) over a != b: relative
  // to the diagonal, down to an absolute floor tied to G's trace (the
  // updates leave noise of an absolute size, which no rotation removes
  // relative to a small eigenvalue)
  auto offdiag = [&]() -> double {
    double mx = 0.0;
    for (int e = tid; e < kSP * kSP; e += 256) {
      const int a = e / kSP, b = e % kSP;
      if (a == b) continue;
      const double v = fabs(S[a][b]), d = sqrt(fabs(S[a][a] * S[b][b])) + floor_abs;
      mx = fmax(mx, d > 0.0 ? v / d : (v > 0.0 ? 1.0 : 0.0));
      if (!(v == v)) mx = 1.0;   // NaN: not converged
    }
    for (int d = 32; d >= 1; d >>= 1) mx = fmax(mx, __shfl_xor(mx, d, 64));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const double r = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    __syncthreads();
    return r;
  };
  const double before = offdiag();
  if (tid == 0) atomicMax(off, (unsigned long long)__double_as_longlong(before));
  double cur = before;
  for (int sw = 0; sw < 10 && cur > kSvdTol * 0.1; ++sw) {   // quadratic: a few sweeps
    for (int k = 0; k < kSP - 1; ++k) {
      if (tid < kSP / 2) {   // the round's rotations (stable symmetric Schur pair)
        int a, b;
        pair_of(kSP, k, tid, a, b);
        const double apq = S[a][b];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (S[b][b] - S[a][a]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        cs[tid] = c;
        sn[tid] = s;
      }
      __syncthreads();
      for (int e = tid; e < (kSP / 2) * kSP; e += 256) {   // rows a, b <- J^T rows
        const int t = e / kSP, col = e % kSP;
        int a, b;
        pair_of(kSP, k, t, a, b);
        const double c = cs[t], s = sn[t], x = S[a][col], y = S[b][col];
        S[a][col] = c * x - s * y;
        S[b][col] = s * x + c * y;
      }
      __syncthreads();
      for (int e = tid; e < (kSP / 2) * kSP; e += 256) {   // columns a, b <- columns J (S and Q)
        const int t = e / kSP, row = e % kSP;
        int a, b;
        pair_of(kSP, k, t, a, b);
        const double c = cs[t], s = sn[t];
        const double x = S[row][a], y = S[row][b];
        S[row][a] = c * x - s * y;
        S[row][b] = s * x + c * y;
        const double u = Q[row][a], v = Q[row][b];
        Q[row][a] = c * u - s * v;
        Q[row][b] = s * u + c * v;
      }
      __syncthreads();
    }
    cur = offdiag();
  }
  double* Qo = Qall + (size_t)blockIdx.x * kSP * kSP;
  for (int e = tid; e < kSP * kSP; e += 256) Qo[e] = Q[e / kSP][e % kSP];
}

// Rows P of M (G, z = 0, or W, z = 1) over columns [64 c, 64 c + 64):
// M[P][cols] <- Q^T M[P][cols], for every pair of the round.
__global__ void __launch_bounds__(256) k_bj_rows(double* __restrict__ G, double* __restrict__ W, int mp, int nb,
                                                 int round, const double* __restrict__ Qall) {
  __shared__ double Qs[kSP][kSP + 1], Ms[kSP][kSP + 1];
  double* M = blockIdx.z == 0 ? G : W;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  int I, J;
  pair_of(nb, round, blockIdx.x, I, J);
  const int c0 = blockIdx.y * kSP;
  const double* Qi = Qall + (size_t)blockIdx.x * kSP * kSP;
  for (int e = tid; e < kSP * kSP; e += 256) {
    const int a = e / kSP, b = e % kSP;
    Qs[a][b] = Qi[e];
    Ms[a][b] = M[(size_t)gidx(I, J, a) * mp + c0 + b];
  }
  __syncthreads();
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int b = 0; b < kSP; ++b) {
    double q[4], x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      q[u] = Qs[b][4 * ty + u];   // (Q^T)[row][b] = Q[b][row]
      x[u] = Ms[b][4 * tx + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fma(q[u], x[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) M[(size_t)gidx(I, J, 4 * ty + u) * mp + c0 + 4 * tx + v] = acc[u][v];
}

// Columns P of G over rows [64 c, 64 c + 64): G[rows][P] <- G[rows][P] Q.
__global__ void __launch_bounds__(256) k_bj_cols(double* __restrict__ G, int mp, int nb, int round,
                                                 const double* __restrict__ Qall) {
  __shared__ double Qs[kSP][kSP + 1], Ms[kSP][kSP + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  int I, J;
  pair_of(nb, round, blockIdx.x, I, J);
  const int r0 = blockIdx.y * kSP;
  const double* Qi = Qall + (size_t)blockIdx.x * kSP * kSP;
  for (int e = tid; e < kSP * kSP; e += 256) {
    const int a = e / kSP, b = e % kSP;
    Qs[a][b] = Qi[e];
    Ms[a][b] = G[(size_t)(r0 + a) * mp + gidx(I, J, b)];
  }
  __syncthreads();
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int b = 0; b < kSP; ++b) {
    double x[4], q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = Ms[4 * ty + u][b];
      q[u] = Qs[b][4 * tx + u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = fma(x[u], q[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) G[(size_t)(r0 + 4 * ty + u) * mp + gidx(I, J, 4 * tx + v)] = acc[u][v];
}

// d[e] = G[e][e], e < m.
__global__ void __launch_bounds__(256) k_diag(const double* __restrict__ G, int mp, int m, double* __restrict__ d) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < m) d[e] = G[(size_t)e * mp + e];
}

// Signs of the output pairs whose v is an eigenvector row (!trans): for
// output i (eigenvector perm[i]): v = W[perm[i]][0 .. m), argmax |v|
// (lowest index on ties) -> s; V[i] = s v (fp32); fac[i] = s / sigma_i (0
// for sigma_i = 0); sigma[i].  One block per output pair.
__global__ void __launch_bounds__(256) k_sign_v(const double* __restrict__ W, int mp, int m,
                                                const int32_t* __restrict__ perm, const double* __restrict__ d,
                                                float* __restrict__ V, float* __restrict__ sigma,
                                                double* __restrict__ fac) {
  __shared__ double bv[4];
  __shared__ int bi[4];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* w = W + (size_t)perm[i] * mp;
  double mv = -1.0;
  int mi = 0;
  for (int k = tid; k < m; k += 256) {
    const double a = fabs(w[k]);
    if (a > mv) { mv = a; mi = k; }   // k increases per thread: the first maximum stays
  }
  for (int dd = 32; dd >= 1; dd >>= 1) {
    const double ov = __shfl_xor(mv, dd, 64);
    const int oi = __shfl_xor(mi, dd, 64);
    if (ov > mv || (ov == mv && oi < mi)) { mv = ov; mi = oi; }
  }
  if (lane == 0) { bv[wave] = mv; bi[wave] = mi; }
  __syncthreads();
  double v0 = bv[0];
  int i0 = bi[0];
  for (int q = 1; q < 4; ++q)
    if (bv[q] > v0 || (bv[q] == v0 && bi[q] < i0)) { v0 = bv[q]; i0 = bi[q]; }
  const double s = w[i0] < 0.0 ? -1.0 : 1.0;
  for (int k = tid; k < m; k += 256) V[(size_t)i * m + k] = (float)(s * w[k]);
  const double sg = sqrt(fmax(d[perm[i]], 0.0));
  if (tid == 0) {
    sigma[i] = (float)sg;
    fac[i] = sg > 0.0 ? s / sg : 0.0;
  }
}

// The derived vectors: Y[i][x] = fac[i] * sum_k W[perm[i]][k] A'(x, k),
// k < m, x < n, with A'(x, k) = A[x][k] (!trans: A [n][m]) or A[k][x]
// (trans: A [m][n]); Y fp32 [r][n].  Block: a 64 x 64 tile of (i, x), fp64
// sums.
__global__ void __launch_bounds__(256) k_derive(const double* __restrict__ W, int mp, const float* __restrict__ A,
                                                int m, int n, int trans, const int32_t* __restrict__ perm,
                                                const double* __restrict__ fac, int r, float* __restrict__ Y) {
  __shared__ double Ws[kSK][kST + 1];
  __shared__ float As[kSK][kST + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int i0 = blockIdx.y * kST, x0 = blockIdx.x * kST;
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int k0 = 0; k0 < m; k0 += kSK) {
    for (int e = tid; e < kSK * kST; e += 256) {
      const int kk = e % kSK, ii = e / kSK;   // along k: a row of W
      const int i = i0 + ii, k = k0 + kk;
      Ws[kk][ii] = (i < r && k < m) ? W[(size_t)perm[i] * mp + k] : 0.0;
    }
    for (int e = tid; e < kSK * kST; e += 256) {
      // !trans: A[x][k], along k; trans: A[k][x], along x
      const int kk = trans ? e / kST : e % kSK, xx = trans ? e % kST : e / kSK;
      const int x = x0 + xx, k = k0 + kk;
      As[kk][xx] = (x < n && k < m) ? (trans ? A[(size_t)k * n + x] : A[(size_t)x * m + k]) : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kSK; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = Ws[k][4 * ty + u];
        b[u] = (double)As[k][4 * tx + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + 4 * ty + u;
    if (i >= r) continue;
    const double f = fac[i];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int x = x0 + 4 * tx + v;
      if (x < n) Y[(size_t)i * n + x] = (float)(f * acc[u][v]);
    }
  }
}

// Signs of the output pairs whose v was derived (trans): argmax |V[i]| over
// n entries (lowest index on ties) -> s; V[i] *= s; U[i] = s W[perm[i]]
// (fp32, m entries); sigma[i].
__global__ void __launch_bounds__(256) k_sign_u(const double* __restrict__ W, int mp, int m, int n,
                                                const int32_t* __restrict__ perm, const double* __restrict__ d,
                                                float* __restrict__ U, float* __restrict__ V,
                                                float* __restrict__ sigma) {
  __shared__ float bv[4];
  __shared__ int bi[4];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* v = V + (size_t)i * n;
  float mv = -1.f;
  int mi = 0;
  for (int k = tid; k < n; k += 256) {
    const float a = fabsf(v[k]);
    if (a > mv) { mv = a; mi = k; }
  }
  for (int dd = 32; dd >= 1; dd >>= 1) {
    const float ov = __shfl_xor(mv, dd, 64);
    const int oi = __shfl_xor(mi, dd, 64);
    if (ov > mv || (ov == mv && oi < mi)) { mv = ov; mi = oi; }
  }
  if (lane == 0) { bv[wave] = mv; bi[wave] = mi; }
  __syncthreads();
  float v0 = bv[0];
  int i0 = bi[0];
  for (int q = 1; q < 4; ++q)
    if (bv[q] > v0 || (bv[q] == v0 && bi[q] < i0)) { v0 = bv[q]; i0 = bi[q]; }
  const float s = v[i0] < 0.f ? -1.f : 1.f;
  __syncthreads();   // every thread has read v[i0] before any flips it
  for (int k = tid; k < n; k += 256) v[k] *= s;
  const double* w = W + (size_t)perm[i] * mp;
  for (int k = tid; k < m; k += 256) U[(size_t)i * m + k] = (float)(s * w[k]);
  if (tid == 0) sigma[i] = (float)sqrt(fmax(d[perm[i]], 0.0));
}

}  // namespace

SvdLayout svd_layout(int32_t out, int32_t in, int32_t r) {
  SvdLayout L{};
  const int m = out < in ? out : in;
  L.m = m;
  L.mp = (int)round_up((size_t)m, kST);
  const size_t mp = (size_t)L.mp;
  const int nb = L.mp / kSB;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, 256);
    return at;
  };
  L.G = take(mp * mp * 8);
  L.W = take(mp * mp * 8);
  L.Q = take((size_t)(nb / 2) * kSP * kSP * 8);
  L.off = take((size_t)kSvdMaxSweeps * 8);
  L.d = take(mp * 8);
  L.fac = take(mp * 8);
  L.perm = take(mp * 4);
  L.flag = take(4);
  L.total = o;
  (void)r;
  return L;
}

int launch_svd(int32_t out, int32_t in, int32_t r, const float* A, float* U, float* sigma, float* V, uint8_t* ws,
               int32_t* sweeps_used, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const SvdLayout L = svd_layout(out, in, r);
  const int m = L.m, mp = L.mp, nb = mp / kSB;
  const int trans = out < in ? 1 : 0;   // G = A A^T: its eigenvectors are the left vectors
  const int n = trans ? in : out;
  double* G = reinterpret_cast<double*>(ws + L.G);
  double* W = reinterpret_cast<double*>(ws + L.W);
  double* Q = reinterpret_cast<double*>(ws + L.Q);
  unsigned long long* off = reinterpret_cast<unsigned long long*>(ws + L.off);
  double* d = reinterpret_cast<double*>(ws + L.d);
  double* fac = reinterpret_cast<double*>(ws + L.fac);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws + L.flag);
  if (sweeps_used) *sweeps_used = 0;
  if (hipMemsetAsync(flag, 0, 4, st) != hipSuccess) return -1;
  const size_t ne = (size_t)mp * mp;
  hipLaunchKernelGGL(k_eye, dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st, W, mp, off, kSvdMaxSweeps);
  hipLaunchKernelGGL(k_gram, dim3((unsigned)(mp / kST), (unsigned)(mp / kST)), dim3(256), 0, st, A, m, n, trans, mp,
                     G, flag);
  uint32_t hflag = 0;
  if (hipMemcpyAsync(&hflag, flag, 4, hipMemcpyDeviceToHost, st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
    return -1;
  if (hflag) return 1;   // a non-finite entry
  // the absolute floor of the convergence test: a tenth of trace(G) (at least
  // lambda_1 / 10), above the rounding noise the updates leave (about 1e-16
  // sqrt(m) lambda_1 relative to the floor's 1e-14 lambda_1 at the tolerance)
  std::vector<double> hd((size_t)m);
  hipLaunchKernelGGL(k_diag, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, G, mp, m, d);
  if (hipMemcpyAsync(hd.data(), d, (size_t)m * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return -1;
  double tr = 0.0;
  for (double v : hd) tr += v;
  const double floor_abs = 0.1 * tr;
  int sw = 0;
  bool conv = false;
  for (; sw < kSvdMaxSweeps && !conv; ++sw) {
    for (int k = 0; k < nb - 1; ++k) {
      hipLaunchKernelGGL(k_bj_eig, dim3((unsigned)(nb / 2)), dim3(256), 0, st, G, mp, nb, k, floor_abs, Q, off + sw);
      hipLaunchKernelGGL(k_bj_rows, dim3((unsigned)(nb / 2), (unsigned)(mp / kSP), 2), dim3(256), 0, st, G, W, mp, nb,
                         k, Q);
      hipLaunchKernelGGL(k_bj_cols, dim3((unsigned)(nb / 2), (unsigned)(mp / kSP)), dim3(256), 0, st, G, mp, nb, k, Q);
    }
    unsigned long long h = 0;
    if (hipMemcpyAsync(&h, off + sw, 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return -1;
    double v;
    memcpy(&v, &h, 8);
    conv = v <= kSvdTol;   // every pair of the sweep was diagonal when it came up
  }
  if (sweeps_used) *sweeps_used = sw;
  if (!conv) return 2;
  // eigenvalues, sorted descending (index order on ties) on the host
  hipLaunchKernelGGL(k_diag, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, G, mp, m, d);
  if (hipMemcpyAsync(hd.data(), d, (size_t)m * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return -1;
  std::vector<int32_t> hp((size_t)m);
  for (int i = 0; i < m; ++i) hp[(size_t)i] = i;
  std::stable_sort(hp.begin(), hp.end(), [&](int32_t a, int32_t b) { return hd[(size_t)a] > hd[(size_t)b]; });
  if (r == 0) return 0;
  std::vector<double> hf((size_t)r);   // (alive until the final synchronization)
  if (hipMemcpyAsync(perm, hp.data(), (size_t)r * 4, hipMemcpyHostToDevice, st) != hipSuccess) return -1;
  const dim3 gd((unsigned)((n + kST - 1) / kST), (unsigned)((r + kST - 1) / kST));
  if (!trans) {   // W rows are v (in = m), U = A v / sigma (out = n)
    hipLaunchKernelGGL(k_sign_v, dim3((unsigned)r), dim3(256), 0, st, W, mp, m, perm, d, V, sigma, fac);
    hipLaunchKernelGGL(k_derive, gd, dim3(256), 0, st, W, mp, A, m, n, 0, perm, fac, r, U);
  } else {   // W rows are u (out = m), V = A^T u / sigma (in = n), then the signs from V
    for (int i = 0; i < r; ++i) {
      const double sg = std::sqrt(std::max(hd[(size_t)hp[(size_t)i]], 0.0));
      hf[(size_t)i] = sg > 0.0 ? 1.0 / sg : 0.0;
    }
    if (hipMemcpyAsync(fac, hf.data(), (size_t)r * 8, hipMemcpyHostToDevice, st) != hipSuccess) return -1;
    hipLaunchKernelGGL(k_derive, gd, dim3(256), 0, st, W, mp, A, m, n, 1, perm, fac, r, V);
    hipLaunchKernelGGL(k_sign_u, dim3((unsigned)r), dim3(256), 0, st, W, mp, m, n, perm, d, U, V, sigma);
  }
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(st) != hipSuccess) return -1;
  return 0;
}

}  // namespace dc

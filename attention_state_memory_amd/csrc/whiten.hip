// Whitening at retrieval (d in {64, 128}; bf16 or float32 rows).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Inferencia Online -- Recuperación: the
// nearest centroid is found by cosine similarity, optionally after a
// whitening transform.  The transform is fit per head on the calibration
// queries X [H, N, d] as x -> W (x - mu): mu the mean, Sigma the population
// covariance plus ridge * trace(Sigma) / d on the diagonal, W = Sigma^-1/2
// (symmetric).  Whitened rows are rounded once (nearest-even) to the row
// type; the lookup then scores them by cosine like unwhitened rows.
//
// Kernels (everything in float64):
//   wh_mean_partial  per (head, row block): column sums of X;
//   wh_mean_final    per head: mu = sum of the block sums / N;
//   wh_cov_partial   per (head, row block): sum of (x - mu)(x - mu)^T over
//                    the block, 16 rows at a time staged in LDS, an 8x8 (d =
//                    128) or 4x4 (d = 64) tile of the d x d sum per thread;
//   wh_invsqrt       one workgroup per head: Sigma from the block sums, the
//                    ridge, then the coupled Newton-Schulz iteration for the
//                    matrix square root (N. J. Higham, "Functions of
//                    Matrices", SIAM 2008, the Newton-Schulz variant of the
//                    Denman-Beavers iteration): with A = Sigma / |Sigma|_F,
//                    Y0 = A, Z0 = I, T = (3I - Z Y) / 2, Y <- Y T, Z <- T Z,
//                    Z converges to A^-1/2 (all eigenvalues of A are in
//                    (0, 1]); W = Z / sqrt(|Sigma|_F), symmetrised;
//   wh_rows          Yw = round(W (y - mu)) for rows y at any head and row
//                    stride: 32 rows x 64 outputs per workgroup on the
//                    float64 MFMA (16x16x4), operands staged in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kCovRows = 16;   // rows staged per pass of wh_cov_partial
constexpr int kGemmK = 16;     // k-slab of the in-workgroup products
constexpr double kConverged = 1e-6;  // |Z Y - I|_F at which the iteration counts as converged

template <typename T>
__device__ __forceinline__ double load_d(const T* p, size_t i) {
  return double(load_elem(p, i));
}

template <typename T>
__device__ __forceinline__ void store_round(T* p, size_t i, double v);
template <>
__device__ __forceinline__ void store_round<uint16_t>(uint16_t* p, size_t i, double v) {
  p[i] = f64_to_bf16_rne(v);
}
template <>
__device__ __forceinline__ void store_round<float>(float* p, size_t i, double v) {
  p[i] = float(v);  // nearest-even
}

__device__ __forceinline__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

}  // namespace

template <typename T>
__global__ void __launch_bounds__(kThreads) wh_mean_partial(WhitenFitArgs a) {
  __shared__ double red[kThreads];
  const int h = blockIdx.x / a.nblk, blk = blockIdx.x % a.nblk;
  const int d = a.d, t = threadIdx.x;
  const int rp = kThreads / d;  // rows in parallel (d divides 256)
  const int dim = t % d, rs = t / d;
  const int64_t r0 = int64_t(a.N) * blk / a.nblk, r1 = int64_t(a.N) * (blk + 1) / a.nblk;
  const T* X = static_cast<const T*>(a.X) + size_t(h) * a.N * d;
  double s = 0.0;
  for (int64_t r = r0 + rs; r < r1; r += rp) s += load_d(X, size_t(r) * d + dim);
  red[t] = s;
  __syncthreads();
  if (t < d) {
    double tot = 0.0;
    for (int j = 0; j < rp; ++j) tot += red[t + j * d];
    a.part_mean[(size_t(h) * a.nblk + blk) * d + t] = tot;
  }
}

__global__ void __launch_bounds__(kThreads) wh_mean_final(WhitenFitArgs a) {
  const int h = blockIdx.x, t = threadIdx.x;
  if (t >= a.d) return;
  double s = 0.0;
  for (int j = 0; j < a.nblk; ++j) s += a.part_mean[(size_t(h) * a.nblk + j) * a.d + t];
  a.mu[size_t(h) * a.d + t] = s / double(a.N);
}

template <typename T, int D>
__global__ void __launch_bounds__(kThreads) wh_cov_partial(WhitenFitArgs a) {
  constexpr int TS = D / 16;
  __shared__ double xs[kCovRows][D];
  __shared__ double mus[D];
  const int h = blockIdx.x / a.nblk, blk = blockIdx.x % a.nblk;
  const int t = threadIdx.x, ti = t / 16, tj = t % 16;
  const int64_t r0 = int64_t(a.N) * blk / a.nblk, r1 = int64_t(a.N) * (blk + 1) / a.nblk;
  const T* X = static_cast<const T*>(a.X) + size_t(h) * a.N * D;
  if (t < D) mus[t] = a.mu[size_t(h) * D + t];
  double acc[TS][TS];
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) acc[i][j] = 0.0;
  __syncthreads();
  for (int64_t base = r0; base < r1; base += kCovRows) {
    for (int e = t; e < kCovRows * D; e += kThreads) {
      const int r = e / D, k = e % D;
      const int64_t row = base + r;
      xs[r][k] = row < r1 ? load_d(X, size_t(row) * D + k) - mus[k] : 0.0;
    }
    __syncthreads();
    for (int r = 0; r < kCovRows; ++r) {
      double u[TS], v[TS];
#pragma unroll
      for (int i = 0; i < TS; ++i) {
        u[i] = xs[r][ti * TS + i];
        v[i] = xs[r][tj * TS + i];
      }
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TS; ++j) acc[i][j] = fma(u[i], v[j], acc[i][j]);
    }
    __syncthreads();
  }
  double* out = a.part_cov + (size_t(h) * a.nblk + blk) * D * D;
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) out[(ti * TS + i) * D + tj * TS + j] = acc[i][j];
}

namespace {

// C = A B for D x D row-major float64 matrices in global memory, computed by
// the whole workgroup; As/Bs are LDS slabs.  Ends with a barrier, so C is
// visible to every thread of the workgroup afterwards.
template <int D>
__device__ void wg_gemm(const double* A, const double* B, double* C, double (*As)[kGemmK + 1],
                        double (*Bs)[D + 1]) {
  constexpr int TS = D / 16;
  const int t = threadIdx.x, ti = t / 16, tj = t % 16;
  double acc[TS][TS];
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) acc[i][j] = 0.0;
  for (int k0 = 0; k0 < D; k0 += kGemmK) {
    for (int e = t; e < D * kGemmK; e += kThreads) {
      As[e / kGemmK][e % kGemmK] = A[(e / kGemmK) * D + k0 + e % kGemmK];
      Bs[e / D][e % D] = B[(k0 + e / D) * D + e % D];
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < kGemmK; ++kk) {
      double u[TS], v[TS];
#pragma unroll
      for (int i = 0; i < TS; ++i) {
        u[i] = As[ti * TS + i][kk];
        v[i] = Bs[kk][tj * TS + i];
      }
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TS; ++j) acc[i][j] = fma(u[i], v[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) C[(ti * TS + i) * D + tj * TS + j] = acc[i][j];
  __threadfence_block();
  __syncthreads();
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(kThreads) wh_invsqrt(WhitenFitArgs a) {
  __shared__ double As[D][kGemmK + 1];
  __shared__ double Bs[kGemmK][D + 1];
  __shared__ double red[4];
  const int h = blockIdx.x, t = threadIdx.x;
  double* buf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) buf[i] = a.mats + (size_t(h) * 4 + i) * D * D;
  // Sigma = (sum of the block sums) / N, into buf[0]; its trace
  const double* pc = a.part_cov + size_t(h) * a.nblk * D * D;
  double tr = 0.0;
  for (int e = t; e < D * D; e += kThreads) {
    double s = 0.0;
    for (int j = 0; j < a.nblk; ++j) s += pc[size_t(j) * D * D + e];
    s /= double(a.N);
    buf[0][e] = s;
    if (e / D == e % D) tr += s;
  }
  tr = block_sum_d(tr, red);
  const double eps = a.ridge * tr / double(D);
  double fro = 0.0;
  for (int e = t; e < D * D; e += kThreads) {
    const double s = buf[0][e] + (e / D == e % D ? eps : 0.0);
    fro += s * s;
  }
  fro = sqrt(block_sum_d(fro, red));
  // Y0 = Sigma_ridged / |.|_F in buf[0], Z0 = I in buf[1]
  const double inv_fro = fro > 0.0 ? 1.0 / fro : 0.0;
  for (int e = t; e < D * D; e += kThreads) {
    const bool diag = e / D == e % D;
    buf[0][e] = (buf[0][e] + (diag ? eps : 0.0)) * inv_fro;
    buf[1][e] = diag ? 1.0 : 0.0;
  }
  __threadfence_block();
  __syncthreads();
  int y = 0, z = 1, p = 2, q = 3;
  double res = INFINITY, prev = INFINITY;
  int it = 0;
  for (; it < a.max_iters; ++it) {
    wg_gemm<D>(buf[z], buf[y], buf[p], As, Bs);  // P = Z Y
    double r2 = 0.0;
    for (int e = t; e < D * D; e += kThreads) {
      const double v = buf[p][e] - (e / D == e % D ? 1.0 : 0.0);
      r2 += v * v;
    }
    prev = res;
    res = sqrt(block_sum_d(r2, red));
    // converged, or stalled at the rounding floor
    if (res < 1e-14 || (res < kConverged && res > 0.5 * prev)) break;
    for (int e = t; e < D * D; e += kThreads)  // T = (3I - P) / 2, in place
      buf[p][e] = (e / D == e % D ? 1.5 : 0.0) - 0.5 * buf[p][e];
    __threadfence_block();
    __syncthreads();
    wg_gemm<D>(buf[y], buf[p], buf[q], As, Bs);  // Y' = Y T
    wg_gemm<D>(buf[p], buf[z], buf[y], As, Bs);  // Z' = T Z (Y no longer needed)
    const int ny = q, nz = y;
    q = z;
    y = ny;
    z = nz;
  }
  // W = Z / sqrt(|Sigma|_F), symmetrised.  An iteration that did not
  // converge (a singular covariance without ridge, a constant corpus) leaves
  // W as NaN, so nothing downstream can use it unnoticed.
  const bool converged = res < kConverged && fro > 0.0;
  const double sc = converged ? 0.5 / sqrt(fro) : NAN;
  double* W = a.W + size_t(h) * D * D;
  for (int e = t; e < D * D; e += kThreads) {
    const int i = e / D, j = e % D;
    W[e] = converged ? (buf[z][i * D + j] + buf[z][j * D + i]) * sc : NAN;
  }
  if (t == 0 && a.resid) a.resid[h] = res;
}

// One workgroup per (head, 32 rows, 64 outputs); wave w owns outputs
// [16 w, 16 w + 16) of the 64 for all 32 rows, as two 16 x 16 tiles on the
// float64 matrix cores (16x16x4 per step, D/4 steps each).  The 32 centred
// rows and each wave's 16 rows of W are first staged in LDS with coalesced
// loads.  Lane l supplies row / output l % 16 and k = 4 s + l / 16 at step s;
// after the last step lane l holds rows l / 16 + 4 r (r = 0..3) of output
// l % 16.
template <typename T, int D>
__global__ void __launch_bounds__(kThreads) wh_rows(WhitenRowsArgs a) {
  constexpr int KL = D / 4;
  constexpr int LD = D + 2;  // LDS row pitch (doubles)
  constexpr int NG = D / 64;  // 64-output groups per head
  __shared__ double wsm[4][16 * LD];
  __shared__ double ysm[32 * LD];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = blockIdx.x % NG;
  const int h = (blockIdx.x / NG) % a.H;
  const int64_t row0 = int64_t(blockIdx.x / NG / a.H) * 32;
  // All staging loads are issued before the first LDS store (one round trip):
  // thread t always covers dim t % D of rows t / D + (256 / D) j, and a row
  // past M reads row M - 1 and stores 0.
  constexpr int YE = 32 * D / kThreads;
  constexpr int WE = 16 * D / 2 / 64;
  const int o0 = g * 64 + w * 16;  // first output of this wave
  const double* W = a.W + (size_t(h) * D + o0) * D;
  double2 wv[WE];
#pragma unroll
  for (int j = 0; j < WE; ++j) wv[j] = *reinterpret_cast<const double2*>(W + 2 * (lane + 64 * j));
  const T* Y = static_cast<const T*>(a.Y);
  const int k_t = t % D, r_t = t / D;
  const double mu_t = a.mu[size_t(h) * D + k_t];
  T yv[YE];  // raw elements: converted only after every load is issued
#pragma unroll
  for (int j = 0; j < YE; ++j) {
    const int64_t row = row0 + r_t + (kThreads / D) * j;
    const int64_t rc = row < a.M ? row : a.M - 1;
    yv[j] = Y[size_t(h * a.head_stride + rc * a.row_stride + k_t)];
  }
#pragma unroll
  for (int j = 0; j < YE; ++j) {
    const int r = r_t + (kThreads / D) * j;
    ysm[r * LD + k_t] = row0 + r < a.M ? load_d(yv, j) - mu_t : 0.0;
  }
#pragma unroll
  for (int j = 0; j < WE; ++j) {
    const int e = 2 * (lane + 64 * j);
    const int r = e / D, k = e % D;
    wsm[w][r * LD + k] = wv[j].x;
    wsm[w][r * LD + k + 1] = wv[j].y;
  }
  __syncthreads();
  const int i = lane % 16, kq = lane / 16;
  f64x4 c0 = {0.0, 0.0, 0.0, 0.0}, c1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
  for (int s = 0; s < KL; ++s) {
    const int k = 4 * s + kq;
    const double b = wsm[w][i * LD + k];
    c0 = __builtin_amdgcn_mfma_f64_16x16x4f64(ysm[i * LD + k], b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f64_16x16x4f64(ysm[(16 + i) * LD + k], b, c1, 0, 0, 0);
  }
  T* Yw = static_cast<T*>(a.Yw);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t ra = row0 + kq + 4 * r, rb = ra + 16;
    if (ra < a.M) store_round(Yw, size_t(h * a.head_stride + ra * a.row_stride + o0 + i), c0[r]);
    if (rb < a.M) store_round(Yw, size_t(h * a.head_stride + rb * a.row_stride + o0 + i), c1[r]);
  }
}

// ---------------------------------------------------------------------------
int whiten_blocks(int H, int N) {
  int nb = (N + 4095) / 4096;
  const int want = (512 + H - 1) / H;
  if (nb > want) nb = want;
  if (nb > 64) nb = 64;
  return nb < 1 ? 1 : nb;
}

size_t whiten_fit_ws_bytes(int H, int N, int d) {
  const int nb = whiten_blocks(H, N);
  return align_up(size_t(H) * nb * d * 8, 256) + align_up(size_t(H) * nb * d * d * 8, 256) +
         align_up(size_t(H) * 4 * d * d * 8, 256);
}

hipError_t launch_whiten_fit(WhitenFitArgs a, int dtype, hipStream_t s) {
  const dim3 blk(kThreads);
  const dim3 parts(unsigned(a.H * a.nblk));
  if (dtype == 0)
    hipLaunchKernelGGL(wh_mean_partial<uint16_t>, parts, blk, 0, s, a);
  else
    hipLaunchKernelGGL(wh_mean_partial<float>, parts, blk, 0, s, a);
  hipLaunchKernelGGL(wh_mean_final, dim3(unsigned(a.H)), blk, 0, s, a);
  if (a.d == 128) {
    if (dtype == 0)
      hipLaunchKernelGGL((wh_cov_partial<uint16_t, 128>), parts, blk, 0, s, a);
    else
      hipLaunchKernelGGL((wh_cov_partial<float, 128>), parts, blk, 0, s, a);
    hipLaunchKernelGGL(wh_invsqrt<128>, dim3(unsigned(a.H)), blk, 0, s, a);
  } else {
    if (dtype == 0)
      hipLaunchKernelGGL((wh_cov_partial<uint16_t, 64>), parts, blk, 0, s, a);
    else
      hipLaunchKernelGGL((wh_cov_partial<float, 64>), parts, blk, 0, s, a);
    hipLaunchKernelGGL(wh_invsqrt<64>, dim3(unsigned(a.H)), blk, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_whiten_rows(const WhitenRowsArgs& a, int dtype, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  const dim3 grid(unsigned((int64_t(a.M) + 31) / 32 * a.H * (a.d / 64)));
  if (a.d == 128) {
    if (dtype == 0)
      hipLaunchKernelGGL((wh_rows<uint16_t, 128>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((wh_rows<float, 128>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (dtype == 0)
      hipLaunchKernelGGL((wh_rows<uint16_t, 64>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((wh_rows<float, 64>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace asmk

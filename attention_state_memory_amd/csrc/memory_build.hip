// Offline memory build of attention-state memory on gfx950: the aggregation
// step, centroid inverse norms, and the plain VALU kernels for k-means
// assignment and prefix states (float32 data and shapes outside the MFMA
// kernels).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Calibración Offline -- Recolección (per query,
// the attention state over the prefix), Agrupamiento (cluster the queries),
// Agregación (centroid = mean of the cluster's queries; the entry's state
// merges the members' states with the online-softmax rule), Eficiencia (a
// long prefix is processed in chunks merged by the same identity).
//
// Aggregation is a counting sort of the queries by cluster followed by the
// per-cluster finalize (mean, cinv, Z-weighted state):
//   K <= kAggLdsMaxK: per (head, chunk of queries) counts in LDS -> per-head
//     scan of the (cluster, chunk) counts (count, offsets) -> scatter (perm)
//     with LDS cursors;
//   larger K: fill(count) -> histogram with global atomics -> per-head scan
//     (offsets, cursor) -> scatter with global atomics.
// Sums run in float64: a bf16 mean is then the float64 mean rounded once to
// bf16, and the member order inside a cluster (set by atomics) does not
// change the result unless a float64 sum is inexact.
#include "common.hpp"
#include "kernels.hpp"
#include "states_generic.hpp"

namespace asmk {

// ---------------------------------------------------------------------------
// inverse norms
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) inv_norms_kernel(int HK, int d, const T* C, float* cinv) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= HK) return;
  double ss = 0.0;
  for (int x = lane; x < d; x += 64) {
    const double c = load_elem(C, size_t(item) * d + x);
    ss = fma(c, c, ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (lane == 0) cinv[item] = ss > 0.0 ? float(1.0 / sqrt(ss)) : 0.0f;
}

hipError_t launch_inv_norms(int dtype, int H, int K, int d, const void* C, float* cinv,
                            hipStream_t s) {
  const int HK = H * K;
  if (HK == 0) return hipSuccess;
  const dim3 grid((HK + 3) / 4);
  if (dtype == 1)
    hipLaunchKernelGGL(inv_norms_kernel<float>, grid, dim3(256), 0, s, HK, d,
                       static_cast<const float*>(C), cinv);
  else
    hipLaunchKernelGGL(inv_norms_kernel<uint16_t>, grid, dim3(256), 0, s, HK, d,
                       static_cast<const uint16_t*>(C), cinv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// aggregation
// ---------------------------------------------------------------------------
__global__ void fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

__global__ void agg_histogram(AggregateArgs a) {
  const int64_t total = int64_t(a.H) * a.N;
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int h = int(t / a.N);
    const int k = a.idx[t];
    if (k >= 0 && k < a.K) atomicAdd(&a.count[size_t(h) * a.K + k], 1);
  }
}

// ---- counting sort with the counters in LDS (K <= kAggLdsMaxK) ---------------
// Workgroup (h, c) counts the members of every cluster among queries
// [c*kAggChunk, (c+1)*kAggChunk) of head h in LDS and stores the counts as
// part[h, c, k].  agg_scan_pass1/2 turn part into exclusive offsets
// (clusters in order, chunks in order within a cluster) and write count and
// offsets;
// agg_scatter_lds then places every query at its cluster's next slot with
// LDS atomics.  The order of the queries inside one (cluster, chunk) is
// unspecified.
__global__ void __launch_bounds__(256) agg_hist_lds(AggregateArgs a, int nch) {
  extern __shared__ int32_t hs[];
  const int h = blockIdx.x / nch, c = blockIdx.x % nch;
  for (int k = threadIdx.x; k < a.K; k += 256) hs[k] = 0;
  __syncthreads();
  const int i0 = c * kAggChunk, i1 = min(a.N, i0 + kAggChunk);
  const int32_t* idx = a.idx + size_t(h) * a.N;
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    const int k = idx[i];
    if (k >= 0 && k < a.K) atomicAdd(&hs[k], 1);
  }
  __syncthreads();
  int32_t* part = a.part + (size_t(h) * nch + c) * a.K;
  for (int k = threadIdx.x; k < a.K; k += 256) part[k] = hs[k];
}

// The scan of the (cluster, chunk) counts in two passes over blocks of 1024
// clusters, one workgroup per (head, block); thread t owns cluster
// 1024*blk + t.  Pass 1 writes each cluster's count, its offset within the
// block and the block's total (kept in `cursor`, unused by this sort).
__device__ __forceinline__ int32_t block_excl_scan_1024(int32_t v, int32_t* wsum, int32_t& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int32_t before = 0;
  total = 0;
  for (int ww = 0; ww < 16; ++ww) {
    if (ww < w) before += wsum[ww];
    total += wsum[ww];
  }
  return before + x - v;
}

__global__ void __launch_bounds__(1024) agg_scan_pass1(AggregateArgs a, int nch, int nkb) {
  __shared__ int32_t wsum[16];
  const int h = blockIdx.x / nkb, blk = blockIdx.x % nkb;
  const int k = blk * 1024 + threadIdx.x;
  const int32_t* part = a.part + size_t(h) * nch * a.K;
  int32_t v = 0;
  if (k < a.K)
    for (int c = 0; c < nch; ++c) v += part[size_t(c) * a.K + k];
  int32_t total;
  const int32_t excl = block_excl_scan_1024(v, wsum, total);
  if (k < a.K) {
    a.count[size_t(h) * a.K + k] = v;
    a.offsets[size_t(h) * (a.K + 1) + k] = excl;
  }
  if (threadIdx.x == 0) a.cursor[size_t(h) * nkb + blk] = total;
}

// Pass 2 adds the totals of the preceding blocks and turns the chunk counts
// into the chunks' first slots.
__global__ void __launch_bounds__(1024) agg_scan_pass2(AggregateArgs a, int nch, int nkb) {
  __shared__ int32_t carry_s, total_s;
  const int h = blockIdx.x / nkb, blk = blockIdx.x % nkb;
  if (threadIdx.x == 0) {
    int32_t c = 0, t = 0;
    for (int b = 0; b < nkb; ++b) {
      const int32_t s = a.cursor[size_t(h) * nkb + b];
      if (b < blk) c += s;
      t += s;
    }
    carry_s = c;
    total_s = t;
  }
  __syncthreads();
  const int k = blk * 1024 + threadIdx.x;
  int32_t* part = a.part + size_t(h) * nch * a.K;
  if (k < a.K) {
    int32_t run = carry_s + a.offsets[size_t(h) * (a.K + 1) + k];
    a.offsets[size_t(h) * (a.K + 1) + k] = run;
    for (int c = 0; c < nch; ++c) {
      const int32_t n = part[size_t(c) * a.K + k];
      part[size_t(c) * a.K + k] = run;
      run += n;
    }
  }
  if (blk == nkb - 1 && threadIdx.x == 0) a.offsets[size_t(h) * (a.K + 1) + a.K] = total_s;
}

__global__ void __launch_bounds__(256) agg_scatter_lds(AggregateArgs a, int nch) {
  extern __shared__ int32_t cur[];
  const int h = blockIdx.x / nch, c = blockIdx.x % nch;
  const int32_t* part = a.part + (size_t(h) * nch + c) * a.K;
  for (int k = threadIdx.x; k < a.K; k += 256) cur[k] = part[k];
  __syncthreads();
  const int i0 = c * kAggChunk, i1 = min(a.N, i0 + kAggChunk);
  const int32_t* idx = a.idx + size_t(h) * a.N;
  int32_t* perm = a.perm + size_t(h) * a.N;
  for (int i = i0 + threadIdx.x; i < i1; i += 256) {
    const int k = idx[i];
    if (k >= 0 && k < a.K) perm[atomicAdd(&cur[k], 1)] = i;
  }
}

// One 1024-thread workgroup per head: exclusive scan of count[h, :].
__global__ void __launch_bounds__(1024) agg_scan(AggregateArgs a) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int h = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int32_t* cnt = a.count + size_t(h) * a.K;
  int32_t* off = a.offsets + size_t(h) * (a.K + 1);
  int32_t* cur = a.cursor + size_t(h) * a.K;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < a.K; base += 1024) {
    const int k = base + t;
    const int32_t v = k < a.K ? cnt[k] : 0;
    int32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int32_t before = carry_s;
    for (int ww = 0; ww < w; ++ww) before += wsum[ww];
    const int32_t excl = before + x - v;
    if (k < a.K) {
      off[k] = excl;
      cur[k] = excl;
    }
    __syncthreads();
    if (t == 1023) carry_s = excl + v;
    __syncthreads();
  }
  if (t == 0) off[a.K] = carry_s;
}

__global__ void agg_scatter(AggregateArgs a) {
  const int64_t total = int64_t(a.H) * a.N;
  for (int64_t t = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int h = int(t / a.N);
    const int i = int(t - int64_t(h) * a.N);
    const int k = a.idx[t];
    if (k >= 0 && k < a.K) {
      const int pos = atomicAdd(&a.cursor[size_t(h) * a.K + k], 1);
      a.perm[size_t(h) * a.N + pos] = i;
    }
  }
}

template <typename T>
__device__ __forceinline__ void store_rounded(T* p, size_t i, double v);
template <>
__device__ __forceinline__ void store_rounded<float>(float* p, size_t i, double v) {
  p[i] = float(v);
}
template <>
__device__ __forceinline__ void store_rounded<uint16_t>(uint16_t* p, size_t i, double v) {
  p[i] = f64_to_bf16_rne(v);
}

// One wave per (head, cluster).  d <= 256: lane owns dims lane + 64*j.
template <typename T>
__global__ void __launch_bounds__(256) agg_finalize(AggregateArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.H * a.K) return;
  const int h = item / a.K, k = item % a.K;
  const int d = a.d;
  const int32_t* off = a.offsets + size_t(h) * (a.K + 1);
  const int beg = off[k];
  const int n = off[k + 1] - beg;
  const int32_t* mem = a.perm + size_t(h) * a.N + beg;
  T* Crow = static_cast<T*>(a.C) + size_t(item) * d;
  const T* X = static_cast<const T*>(a.X) + size_t(h) * a.N * d;

  double cval[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = lane + 64 * j;
    cval[j] = x < d ? double(load_elem(Crow, x)) : 0.0;
  }
  if (n > 0) {
    double sum[4] = {0.0, 0.0, 0.0, 0.0};
    for (int m = 0; m < n; ++m) {
      const size_t row = size_t(mem[m]) * d;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = lane + 64 * j;
        if (x < d) sum[j] += double(load_elem(X, row + x));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane + 64 * j;
      if (x < d) {
        store_rounded<T>(Crow, x, sum[j] / double(n));
        cval[j] = double(load_elem(Crow, x));
      }
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) ss = fma(cval[j], cval[j], ss);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  if (lane == 0) a.cinv[item] = ss > 0.0 ? float(1.0 / sqrt(ss)) : 0.0f;

  if (a.Abar == nullptr) return;
  float* ab = a.Abar + size_t(item) * d;
  const float* LSE = a.LSE + size_t(h) * a.N;
  const float* A = a.A + size_t(h) * a.N * d;
  float mx = -INFINITY;
  for (int m = lane; m < n; m += 64) mx = fmaxf(mx, LSE[mem[m]]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if (n == 0 || mx == -INFINITY) {
    for (int x = lane; x < d; x += 64) ab[x] = 0.0f;
    if (lane == 0) a.LSEbar[item] = -INFINITY;
    return;
  }
  double z = 0.0, acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int m = 0; m < n; ++m) {
    const int i = mem[m];
    const float li = LSE[i];
    if (li == -INFINITY) continue;
    const double wgt = exp(double(li) - double(mx));
    z += wgt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane + 64 * j;
      if (x < d) acc[j] = fma(wgt, double(A[size_t(i) * d + x]), acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = lane + 64 * j;
    if (x < d) ab[x] = float(acc[j] / z);
  }
  if (lane == 0) a.LSEbar[item] = float(double(mx) + log(z) - log(double(n)));
}

// bf16 queries with d in {64, 128}: one group of D/8 lanes per (head,
// cluster), 64*8/D clusters per wave, so that one wave's three dependent
// memory rounds (member range, member list, member rows) serve several
// clusters at once.  Lane `sub` of a group owns dims 8*sub .. 8*sub+7 of
// the cluster: it sums them over all members in float64 (eight member rows
// in flight), rounds the mean once, and for the states weighs the members'
// a rows (two 16-byte pieces per lane) by Z.  The mean step without states
// is its own instantiation (kStates = false): it needs 70 registers instead
// of 106, so more waves per SIMD overlap the dependent rounds.
template <int D, bool kStates>
__global__ void __launch_bounds__(256) agg_finalize_bf16(AggregateArgs a) {
  constexpr int LG = D / 8;   // lanes per cluster
  constexpr int NG = 64 / LG;  // clusters per wave
  constexpr int XB = 8;        // member rows in flight per group
  const int lane = threadIdx.x & 63;
  const int g = lane / LG, sub = lane % LG, g0 = g * LG;
  const int64_t item = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * NG + g;
  const bool live = item < int64_t(a.H) * a.K;
  const int64_t it = live ? item : 0;
  const int h = int(it / a.K);
  const int32_t* off = a.offsets + size_t(h) * (a.K + 1) + (it - int64_t(h) * a.K);
  const int beg = off[0];
  const int n = live ? off[1] - beg : 0;
  const int32_t* mem = a.perm + size_t(h) * a.N + beg;
  const auto rx = make_rsrc(static_cast<const uint16_t*>(a.X) + size_t(h) * a.N * D, uint32_t(a.N) * D * 2);
  const int x_oob = int(uint32_t(a.N) * D * 2);
  uint16_t* Crow = static_cast<uint16_t*>(a.C) + size_t(it) * D + 8 * sub;

  // ---- centroid: float64 sum of the members, one rounding to bf16
  double c[8];
  if (n > 0) {
    double sum[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    for (int M0 = 0; M0 < n; M0 += 4 * LG) {
      // the member indices of up to four chunks of LG members load in one
      // round; lane `sub` holds member M0 + c*LG + sub of chunk c
      int ids[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) ids[c] = M0 + c * LG + sub < n ? mem[M0 + c * LG + sub] : 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int m0 = M0 + c * LG;
        if (m0 >= n) break;
        const int cnt = min(LG, n - m0);
        for (int b0 = 0; b0 < cnt; b0 += XB) {
          u32x4 v[XB];
#pragma unroll
          for (int j = 0; j < XB; ++j) {
            const int mm = b0 + j;
            const int row = __shfl(ids[c], g0 + (mm & (LG - 1)), 64);
            // members past cnt read from past the buffer end: zeros, no traffic
            v[j] = buf16(rx, mm < cnt ? (row * D + 8 * sub) * 2 : x_oob, 0);
          }
#pragma unroll
          for (int j = 0; j < XB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sum[2 * e] += double(bf16_lo(v[j][e]));
              sum[2 * e + 1] += double(bf16_hi(v[j][e]));
            }
        }
      }
    }
    u32x4 packed;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t lo = f64_to_bf16_rne(sum[2 * e] / double(n));
      const uint16_t hi = f64_to_bf16_rne(sum[2 * e + 1] / double(n));
      packed[e] = uint32_t(lo) | (uint32_t(hi) << 16);
      c[2 * e] = double(bf16_lo(packed[e]));
      c[2 * e + 1] = double(bf16_hi(packed[e]));
    }
    *reinterpret_cast<u32x4*>(Crow) = packed;
  } else {
    const u32x4 packed = *reinterpret_cast<const u32x4*>(Crow);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[2 * e] = double(bf16_lo(packed[e]));
      c[2 * e + 1] = double(bf16_hi(packed[e]));
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fma(c[e], c[e], ss);
#pragma unroll
  for (int m = 1; m < LG; m <<= 1) ss += __shfl_xor(ss, m, 64);
  if (live && sub == 0) a.cinv[it] = ss > 0.0 ? float(1.0 / sqrt(ss)) : 0.0f;

  if (!kStates || !live) return;
  // ---- state: Z-weighted mean of the members' a, mean of their Z
  float* ab = a.Abar + size_t(it) * D + 8 * sub;
  const float* LSE = a.LSE + size_t(h) * a.N;
  const auto ra = make_rsrc(a.A + size_t(h) * a.N * D, uint32_t(a.N) * D * 4);
  const int a_oob = int(uint32_t(a.N) * D * 4);
  float mx = -INFINITY;
  for (int m = sub; m < n; m += LG) mx = fmaxf(mx, LSE[mem[m]]);
#pragma unroll
  for (int m = 1; m < LG; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if (n == 0 || mx == -INFINITY) {
    reinterpret_cast<f32x4*>(ab)[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    reinterpret_cast<f32x4*>(ab)[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (sub == 0) a.LSEbar[it] = -INFINITY;
    return;
  }
  double z = 0.0, acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int m0 = 0; m0 < n; m0 += LG) {
    const int cnt = min(LG, n - m0);
    const int myi = sub < cnt ? mem[m0 + sub] : 0;
    const float li = sub < cnt ? LSE[myi] : -INFINITY;
    const double wl = li == -INFINITY ? 0.0 : exp(double(li) - double(mx));
    z += wl;
    for (int b0 = 0; b0 < cnt; b0 += XB / 2) {
      u32x4 v[XB / 2][2];
#pragma unroll
      for (int j = 0; j < XB / 2; ++j) {
        const int mm = b0 + j;
        const int row = __shfl(myi, g0 + (mm & (LG - 1)), 64);
        const int voff = mm < cnt ? (row * D + 8 * sub) * 4 : a_oob;
        v[j][0] = buf16(ra, voff, 0);
        v[j][1] = buf16(ra, voff, 16);
      }
#pragma unroll
      for (int j = 0; j < XB / 2; ++j) {
        const int mm = b0 + j;
        const double wgt = __shfl(wl, g0 + (mm & (LG - 1)), 64);  // 0 past cnt
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] = fma(wgt, double(__uint_as_float(v[j][0][e])), acc[e]);
          acc[4 + e] = fma(wgt, double(__uint_as_float(v[j][1][e])), acc[4 + e]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LG; m <<= 1) z += __shfl_xor(z, m, 64);
  f32x4 o0, o1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o0[e] = float(acc[e] / z);
    o1[e] = float(acc[4 + e] / z);
  }
  reinterpret_cast<f32x4*>(ab)[0] = o0;
  reinterpret_cast<f32x4*>(ab)[1] = o1;
  if (sub == 0) a.LSEbar[it] = float(double(mx) + log(z) - log(double(n)));
}

// ---------------------------------------------------------------------------
// the entry table grouped by super (two-level index): row i of head h is
// entry members[h, i], copied 16 bytes per thread; cginv follows
// ---------------------------------------------------------------------------
template <int ES>  // element size in bytes
__global__ void __launch_bounds__(256) index_group_rows_kernel(int H, int K, int d, const char* C,
                                                               const float* cinv, const int32_t* members,
                                                               char* Cg, float* cginv) {
  const int pieces = d * ES / 16;  // d * ES is a multiple of 16
  const int64_t total = int64_t(H) * K * pieces;
  for (int64_t x = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; x < total;
       x += int64_t(gridDim.x) * blockDim.x) {
    const int64_t row = x / pieces;
    const int part = int(x - row * pieces);
    const int64_t h = row / K;
    const int e = members[row];
    const bool ok = e >= 0 && e < K;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4*>(C + (h * K + e) * d * ES + part * 16);
    *reinterpret_cast<u32x4*>(Cg + row * d * ES + part * 16) = v;
    if (part == 0) cginv[row] = ok ? cinv[h * K + e] : 0.0f;
  }
}

hipError_t launch_index_group_rows(int dtype, int H, int K, int d, const void* C, const float* cinv,
                                   const int32_t* members, void* Cg, float* cginv, hipStream_t s) {
  const int es = dtype == 0 ? 2 : 4;
  const int64_t total = int64_t(H) * K * (d * es / 16);
  if (total == 0) return hipSuccess;
  const dim3 grid(unsigned((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536));
  if (es == 2)
    hipLaunchKernelGGL(index_group_rows_kernel<2>, grid, dim3(256), 0, s, H, K, d,
                       static_cast<const char*>(C), cinv, members, static_cast<char*>(Cg), cginv);
  else
    hipLaunchKernelGGL(index_group_rows_kernel<4>, grid, dim3(256), 0, s, H, K, d,
                       static_cast<const char*>(C), cinv, members, static_cast<char*>(Cg), cginv);
  return hipGetLastError();
}

hipError_t launch_aggregate(const AggregateArgs& a, int dtype, hipStream_t s) {
  const int64_t HK = int64_t(a.H) * a.K, HN = int64_t(a.H) * a.N;
  if (HK == 0) return hipSuccess;
  auto grid_for = [](int64_t n) { return dim3(unsigned((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536)); };
  if (a.part != nullptr && a.K <= kAggLdsMaxK && a.N > 0) {
    const int nch = agg_chunks(a.N);
    const dim3 cgrid(unsigned(int64_t(a.H) * nch));
    const size_t lds = size_t(a.K) * sizeof(int32_t);
    const int nkb = (a.K + 1023) / 1024;
    hipLaunchKernelGGL(agg_hist_lds, cgrid, dim3(256), lds, s, a, nch);
    hipLaunchKernelGGL(agg_scan_pass1, dim3(unsigned(a.H * nkb)), dim3(1024), 0, s, a, nch, nkb);
    hipLaunchKernelGGL(agg_scan_pass2, dim3(unsigned(a.H * nkb)), dim3(1024), 0, s, a, nch, nkb);
    hipLaunchKernelGGL(agg_scatter_lds, cgrid, dim3(256), lds, s, a, nch);
  } else {
    hipLaunchKernelGGL(fill_i32, grid_for(HK), dim3(256), 0, s, a.count, HK, 0);
    if (HN > 0) hipLaunchKernelGGL(agg_histogram, grid_for(HN), dim3(256), 0, s, a);
    hipLaunchKernelGGL(agg_scan, dim3(a.H), dim3(1024), 0, s, a);
    if (HN > 0) hipLaunchKernelGGL(agg_scatter, grid_for(HN), dim3(256), 0, s, a);
  }
  const dim3 fgrid(unsigned((HK + 3) / 4));
  const bool fits = int64_t(a.N) * a.d * 4 < (int64_t(1) << 31);
  // the bf16 kernel serves 64*8/d clusters per wave, four waves per block
  const int64_t cpb = int64_t(4) * (64 * 8 / (a.d > 0 ? a.d : 1));
  const dim3 ggrid(unsigned((HK + cpb - 1) / cpb));
  const bool states = a.Abar != nullptr;
  if (dtype == 0 && a.d == 128 && fits) {
    if (states) hipLaunchKernelGGL((agg_finalize_bf16<128, true>), ggrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((agg_finalize_bf16<128, false>), ggrid, dim3(256), 0, s, a);
  } else if (dtype == 0 && a.d == 64 && fits) {
    if (states) hipLaunchKernelGGL((agg_finalize_bf16<64, true>), ggrid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((agg_finalize_bf16<64, false>), ggrid, dim3(256), 0, s, a);
  } else if (dtype == 1) {
    hipLaunchKernelGGL(agg_finalize<float>, fgrid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(agg_finalize<uint16_t>, fgrid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// plain VALU k-means assignment: one wave per query
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) assign_generic(AssignArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.H * a.N) return;
  const int h = item / a.N;
  const int d = a.d;
  const T* X = static_cast<const T*>(a.X);
  const T* C = static_cast<const T*>(a.C) + size_t(h) * a.K * d;
  const float* ci = a.cinv + size_t(h) * a.K;
  float qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = lane + 64 * j;
    qv[j] = x < d ? load_elem(X, size_t(item) * d + x) : 0.0f;
  }
  uint64_t best = 0;
  for (int k = 0; k < a.K; ++k) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane + 64 * j;
      if (x < d) s = fmaf(qv[j], load_elem(C, size_t(k) * d + x), s);
    }
    s = wave_sum(s);
    best = umax64(best, argmax_key(s * ci[k], uint32_t(k)));
  }
  if (lane == 0) {
    a.idx[item] = int32_t(key_index(best));
    if (a.best) a.best[item] = key_score(best);
  }
}

hipError_t launch_assign_generic(const AssignArgs& a, int dtype, hipStream_t s) {
  const int64_t HN = int64_t(a.H) * a.N;
  if (HN == 0) return hipSuccess;
  const dim3 grid(unsigned((HN + 3) / 4));
  if (dtype == 1)
    hipLaunchKernelGGL(assign_generic<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(assign_generic<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// plain VALU prefix states: one wave per (query head, query)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) states_generic(StatesArgs a) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.Hq * a.N) return;
  states_one_query<T>(a, item / a.N, item % a.N);
}

hipError_t launch_states_generic(const StatesArgs& a, int dtype, hipStream_t s) {
  const int64_t HN = int64_t(a.Hq) * a.N;
  if (HN == 0) return hipSuccess;
  const dim3 grid(unsigned((HN + 3) / 4));
  if (dtype == 1)
    hipLaunchKernelGGL(states_generic<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(states_generic<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace asmk

// Two-level (hierarchical) retrieval for the decode step (bf16, d in {64, 128}).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Inferencia Online -- Recuperación (nearest
// memory entry by cosine) and Complejidad (the lookup grows with the
// logarithm of the memory size through a hierarchical index).  The index has
// two levels: the entries of a head are clustered into S super-centroids
// (asm_build_index).  A query scores the S supers, probes the p best
// non-empty ones and takes the entry of highest cosine among their members;
// probing every super is the flat search.
//
// One workgroup per (sequence, query head):
//   1. the query goes to LDS as float32;
//   2. each thread scores up to four supers (a dot product over its 16-byte
//      row pieces against the query in LDS) into (score, index) keys; empty
//      supers get no key;
//   3. p rounds of a block-wide maximum pick the probes (lowest index on
//      exact ties);
//   4. the members of the probes are scored in one flattened loop and the
//      block-wide maximum key, the entry of highest score and lowest index,
//      is written where the flat search writes its unit keys (one unit per
//      head), so the attention and merge kernels of the flat path follow
//      unchanged.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

namespace {

constexpr int kThreads = 256;
constexpr int kSupersPerThread = 4;

// q . row over D bf16 values, the query in LDS as float32
template <int D>
__device__ __forceinline__ float dot_row(const uint16_t* row, const float* qs) {
  u32x4 v[D / 8];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) v[c] = ld16(row + 8 * c);
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(v[c][e]), qs[8 * c + 2 * e], acc);
      acc = fmaf(bf16_hi(v[c][e]), qs[8 * c + 2 * e + 1], acc);
    }
  return acc;
}

// block-wide maximum of one key per thread (all threads take part)
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint64_t m = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
  __syncthreads();
  return m;
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(kThreads) hier_lookup_kernel(HierArgs a) {
  __shared__ float qs[D];
  __shared__ uint64_t red[4];
  __shared__ int32_t probe[kHierMaxProbes];
  __shared__ int32_t pbeg[kHierMaxProbes + 1];
  __shared__ int32_t poff[kHierMaxProbes];
  const int t = threadIdx.x;
  const int item = blockIdx.x;  // b * Hq + h
  const int b = item / a.Hq, h = item % a.Hq;

  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + size_t(item) * D;
  if (t < D) qs[t] = load_elem(qp, t);
  __syncthreads();

  const uint16_t* SC = static_cast<const uint16_t*>(a.SC) + size_t(h) * a.S * D;
  const float* scinv = a.scinv + size_t(h) * a.S;
  const int32_t* off = a.offsets + size_t(h) * (a.S + 1);
  uint64_t sk[kSupersPerThread];
#pragma unroll
  for (int i = 0; i < kSupersPerThread; ++i) {
    const int s = t + kThreads * i;
    sk[i] = 0ull;
    if (s < a.S && off[s + 1] > off[s])
      sk[i] = argmax_key(dot_row<D>(SC + size_t(s) * D, qs) * scinv[s], uint32_t(s));
  }

  // probes: p rounds of the block-wide maximum; the owner drops the winner
  int np = 0;
  for (int r = 0; r < a.p; ++r) {
    uint64_t m = sk[0];
#pragma unroll
    for (int i = 1; i < kSupersPerThread; ++i) m = umax64(m, sk[i]);
    const uint64_t best = block_max_u64(m, red);
    if (best == 0ull) break;  // no non-empty super left
#pragma unroll
    for (int i = 0; i < kSupersPerThread; ++i)
      if (sk[i] == best) sk[i] = 0ull;
    if (t == 0) probe[r] = int32_t(key_index(best));
    np = r + 1;
  }
  if (t == 0) {
    int acc = 0;
    for (int r = 0; r < np; ++r) {
      const int s = probe[r];
      poff[r] = off[s];
      pbeg[r] = acc;
      acc += off[s + 1] - off[s];
    }
    pbeg[np] = acc;
  }
  __syncthreads();

  // the probed supers' members, flattened over the probes
  const uint16_t* C = static_cast<const uint16_t*>(a.C) + size_t(h) * a.K * D;
  const float* cinv = a.cinv + size_t(h) * a.K;
  const int32_t* mem = a.members + size_t(h) * a.K;
  const int total = pbeg[np];
  uint64_t best = 0ull;
  for (int j = t; j < total; j += kThreads) {
    int r = 0;
    while (pbeg[r + 1] <= j) ++r;
    const int e = mem[poff[r] + (j - pbeg[r])];
    best = umax64(best, argmax_key(dot_row<D>(C + size_t(e) * D, qs) * cinv[e], uint32_t(e)));
  }
  best = block_max_u64(best, red);
  if (t == 0) a.keys[size_t(h) * a.B + b] = best;
  if (a.probes_out != nullptr && t < a.p)
    a.probes_out[size_t(item) * a.p + t] = t < np ? probe[t] : -1;
}

bool hier_fast_path(int dtype, int d) { return dtype == 0 && (d == 64 || d == 128); }

hipError_t launch_hier_lookup(const HierArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.B * a.Hq));
  if (a.d == 128)
    hipLaunchKernelGGL(hier_lookup_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(hier_lookup_kernel<64>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace asmk

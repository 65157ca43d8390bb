// Two-level (hierarchical) retrieval for the decode step (bf16, d in {64, 128}):
// the per-workgroup lookup, run by the lookup blocks of decode_fast_main_hier.
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
// One 512-thread workgroup per (sequence, query head, probe rank r), r < p:
//   1. the query goes to LDS as float32;
//   2. each thread scores up to two supers (a dot product over its 16-byte
//      row pieces against the query in LDS) into (score, index) keys, kept
//      in LDS; empty supers get no key;
//   3. each thread counts, for its supers, how many keys are larger: the
//      super of rank r is this workgroup's probe (ranks are unique: keys
//      carry the index, lowest index first on exact score ties);
//   4. the probe's members are scored and the block-wide maximum key, the
//      member of highest score and lowest index, is written as unit r of
//      (head, sequence) where the flat search writes its unit keys; with the
//      table grouped by super (Cg, cginv), the member rows sit at the
//      probe's member positions, so they load in the same round as the
//      member indices instead of after them.  The
//      flat path's merge kernel reduces the p units to the entry, and its
//      attention kernel runs unchanged with scoring switched off.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

namespace hier {

// NT: the workgroup size of the decode main grid the lookup runs in
template <int NT>
constexpr int supers_per_thread() { return (kHierMaxSupers + NT - 1) / NT; }

// q . row over D bf16 values held in registers, the query in LDS as float32
template <int D>
__device__ __forceinline__ float dot_regs(const u32x4 (&v)[D / 8], const float* qs) {
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

// q . row over D bf16 values in memory
template <int D>
__device__ __forceinline__ float dot_row(const uint16_t* row, const float* qs) {
  u32x4 v[D / 8];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) v[c] = ld16(row + 8 * c);
  return dot_regs<D>(v, qs);
}

// block-wide maximum of one key per thread (all NT threads take part)
template <int NT>
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t m = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = umax64(m, red[i]);
  __syncthreads();
  return m;
}

}  // namespace hier

// The lookup of one workgroup of NT threads (block index blk of the lookup
// grid).
template <int D, int NT>
__device__ __forceinline__ void hier_lookup_block(const HierArgs& a, int blk) {
  static_assert(NT >= 128 && NT % 64 == 0, "the query load needs a thread per dimension");
  constexpr int kSupersPerThread = hier::supers_per_thread<NT>();
  __shared__ float qs[D];
  __shared__ uint64_t keys_s[kHierMaxSupers];
  __shared__ uint64_t red[NT / 64];
  __shared__ int32_t probe_s;
  const int t = threadIdx.x;
  const int r = blk % a.p;        // probe rank of this workgroup
  const int item = blk / a.p;     // b * Hq + h
  const int b = item / a.Hq, h = item % a.Hq;

  const uint16_t* SC = static_cast<const uint16_t*>(a.SC) + size_t(h) * a.S * D;
  const float* scinv = a.scinv + size_t(h) * a.S;
  const int32_t* off = a.offsets + size_t(h) * (a.S + 1);
  // The thread's first super (its row, inverse norm and member range) does
  // not depend on the query: it loads beside the query, in the same round.
  u32x4 row0[D / 8];
  float si0 = 0.0f;
  int ob0 = 0, oe0 = 0;
  if (t < a.S) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c) row0[c] = ld16(SC + size_t(t) * D + 8 * c);
    si0 = scinv[t];
    ob0 = off[t];
    oe0 = off[t + 1];
  }
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + size_t(item) * D;
  if (t < D) qs[t] = load_elem(qp, t);
  if (t == 0) probe_s = -1;
  __syncthreads();

  uint64_t sk[kSupersPerThread];
#pragma unroll
  for (int i = 0; i < kSupersPerThread; ++i) {
    const int s = t + NT * i;
    sk[i] = 0ull;
    if (i == 0) {
      if (s < a.S && oe0 > ob0) sk[0] = argmax_key(hier::dot_regs<D>(row0, qs) * si0, uint32_t(s));
    } else if (s < a.S && off[s + 1] > off[s]) {
      sk[i] = argmax_key(hier::dot_row<D>(SC + size_t(s) * D, qs) * scinv[s], uint32_t(s));
    }
    if (s < a.S) keys_s[s] = sk[i];
  }
  __syncthreads();
  // rank of each of this thread's supers among the non-empty ones
#pragma unroll
  for (int i = 0; i < kSupersPerThread; ++i) {
    if (sk[i] == 0ull) continue;
    int rank = 0;
    for (int s2 = 0; s2 < a.S; ++s2) rank += keys_s[s2] > sk[i] ? 1 : 0;
    if (rank == r) probe_s = int32_t(key_index(sk[i]));
  }
  __syncthreads();
  const int probe = probe_s;

  uint64_t best = 0ull;
  if (probe >= 0) {
    const uint16_t* C = static_cast<const uint16_t*>(a.C) + size_t(h) * a.K * D;
    const float* cinv = a.cinv + size_t(h) * a.K;
    const int o0 = off[probe];
    const int32_t* mem = a.members + size_t(h) * a.K + o0;
    const int n = off[probe + 1] - o0;
    if (a.Cg != nullptr) {
      const uint16_t* Cg = static_cast<const uint16_t*>(a.Cg) + (size_t(h) * a.K + o0) * D;
      const float* cg = a.cginv + size_t(h) * a.K + o0;
      for (int j = t; j < n; j += NT)
        best = umax64(best, argmax_key(hier::dot_row<D>(Cg + size_t(j) * D, qs) * cg[j], uint32_t(mem[j])));
    } else {
      for (int j = t; j < n; j += NT) {
        const int e = mem[j];
        best = umax64(best, argmax_key(hier::dot_row<D>(C + size_t(e) * D, qs) * cinv[e], uint32_t(e)));
      }
    }
  }
  best = hier::block_max_u64<NT>(best, red);
  if (t == 0) {
    a.keys[(size_t(h) * a.B + b) * a.p + r] = best;
    if (a.probes_out != nullptr) a.probes_out[size_t(item) * a.p + r] = probe;
  }
}

}  // namespace asmk

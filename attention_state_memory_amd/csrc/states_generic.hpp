// Prefix attention states of one (query head, query) by one wave, on the
// float32 VALU with inputs read as stored (bf16 or float32): the plain path
// of asm_build_states, and the fallback of its MFMA kernel when a bf16 value
// is too large for the fp16 value products.
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Calibración Offline -- Recolección (the
// attention state of each calibration query over the prefix) and Eficiencia
// (chunks computed independently and merged by the online-softmax identity).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

// (l1, a1) <- merge((l1, a1), (l2, a2)); lane-local pieces of a d-vector
__device__ __forceinline__ void merge_state(float& l1, float* a1, float l2, const float* a2) {
  const float M = fmaxf(l1, l2);
  if (M == -INFINITY) return;
  const float w1 = l1 == -INFINITY ? 0.0f : expf(l1 - M);
  const float w2 = l2 == -INFINITY ? 0.0f : expf(l2 - M);
  const float z = w1 + w2;
#pragma unroll
  for (int j = 0; j < 4; ++j) a1[j] = (w1 * a1[j] + w2 * a2[j]) / z;
  l1 = M + logf(z);
}

// Query q of head h (item = h * N + q); d <= 256, lane owns dims lane + 64 j.
template <typename T>
__device__ __forceinline__ void states_one_query(const StatesArgs& a, int h, int q) {
  const int lane = threadIdx.x & 63;
  const size_t item = size_t(h) * a.N + q;
  const int g = h / (a.Hq / a.Hkv);
  const int d = a.d;
  const T* Q = static_cast<const T*>(a.Q);
  const T* Kg = static_cast<const T*>(a.Kp) + size_t(g) * a.L * d;
  const T* Vg = static_cast<const T*>(a.Vp) + size_t(g) * a.L * d;
  float qv[4], ra[4];
  float rl = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = lane + 64 * j;
    qv[j] = x < d ? load_elem(Q, item * d + x) : 0.0f;
    ra[j] = (a.accumulate && x < d) ? a.A[item * d + x] : 0.0f;
  }
  if (a.accumulate) rl = a.LSE[item];
  for (int c = 0; c < a.nc; ++c) {
    const int lo = c * a.chunk, hi = min(a.L, lo + a.chunk);
    float m = -INFINITY, l = 0.0f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t = lo; t < hi; ++t) {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = lane + 64 * j;
        if (x < d) s = fmaf(qv[j], load_elem(Kg, size_t(t) * d + x), s);
      }
      s = wave_sum(s) * a.scale2;
      const float mn = fmaxf(m, s);
      const float al = __builtin_amdgcn_exp2f(m - mn);
      const float p = __builtin_amdgcn_exp2f(s - mn);
      l = l * al + p;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = lane + 64 * j;
        const float v = x < d ? load_elem(Vg, size_t(t) * d + x) : 0.0f;
        acc[j] = fmaf(p, v, acc[j] * al);
      }
      m = mn;
    }
    float ca[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ca[j] = acc[j] / l;
    const float cl = (m + log2f(l)) * ASM_LN2;
    if (a.A_chunks) {
      const size_t row = size_t(c) * a.Hq * a.N + item;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = lane + 64 * j;
        if (x < d) a.A_chunks[row * d + x] = ca[j];
      }
      if (lane == 0) a.LSE_chunks[row] = cl;
    }
    merge_state(rl, ra, cl, ca);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = lane + 64 * j;
    if (x < d) a.A[item * d + x] = rl == -INFINITY ? 0.0f : ra[j];
  }
  if (lane == 0) a.LSE[item] = rl;
}

}  // namespace asmk

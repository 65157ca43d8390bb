// Decode step of attention-state memory on gfx950.
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Inferencia Online -- Recuperación (nearest
// centroid by cosine) and Fusión (merge the retrieved state with the query's
// attention over the non-prefix tokens by the online-softmax identity).
//
// This file holds the plain VALU path of the decode step (float32 inputs,
// head dims other than 64/128, GQA groups other than 1/2/4/8); the MFMA path
// is in decode_fast.hip.  Three launches on the caller's stream:
//   score_generic         one thread per centroid, one 64-bit (score, index)
//                         key per (head, 256-centroid tile, sequence);
//   attn_generic          one workgroup per (sequence, kv head, token split),
//                         one wave per query head, online softmax over the
//                         split, one partial state per (b, h, split);
//   decode_combine_split  one wave per (b, h): index from the keys, gather,
//                         merge with the split partials, write the outputs.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

// ---------------------------------------------------------------------------
// combine: index, gather, merge
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_combine_split(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.B * a.Hq) return;
  const int b = item / a.Hq, h = item % a.Hq;
  const int D = a.d;
  uint64_t best = 0;
  for (int t = lane; t < a.score_tiles; t += 64)
    best = umax64(best, a.keys[(size_t(h) * a.score_tiles + t) * a.B + b]);
  best = wave_max_u64(best);
  const uint32_t k = key_index(best);
  if (lane == 0 && a.out_idx) a.out_idx[item] = int32_t(k);
  float* o = a.out + size_t(item) * D;
  const int n = a.kv_len[b];
  const int64_t st = a.kv_start[b];
  if (n < 0 || n > a.max_kv_len || st < 0 || st + n > a.kv_capacity || k >= uint32_t(a.K)) {
    for (int dd = lane; dd < D; dd += 64) o[dd] = NAN;
    if (lane == 0 && a.out_lse) a.out_lse[item] = NAN;
    return;
  }
  const float lm = a.LSEbar[size_t(h) * a.K + k];
  const float* am = a.Abar + (size_t(h) * a.K + k) * D;
  const int ns = n > 0 ? (n + a.split_tok - 1) / a.split_tok : 0;
  const float* pl = a.part_lse + size_t(item) * a.S_max;
  const float* pa = a.part_a + size_t(item) * a.S_max * D;
  float M = lm;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pl[s]);
  if (M == -INFINITY) {
    for (int dd = lane; dd < D; dd += 64) o[dd] = 0.0f;
    if (lane == 0 && a.out_lse) a.out_lse[item] = -INFINITY;
    return;
  }
  const float wm = lm == -INFINITY ? 0.0f : expf(lm - M);
  float Z = wm;
  for (int s = 0; s < ns; ++s) Z += expf(pl[s] - M);
  const float inv = 1.0f / Z;
  for (int dd = lane; dd < D; dd += 64) {
    float v = wm > 0.0f ? wm * am[dd] : 0.0f;
    for (int s = 0; s < ns; ++s) v = fmaf(expf(pl[s] - M), pa[size_t(s) * D + dd], v);
    o[dd] = v * inv;
  }
  if (lane == 0 && a.out_lse) a.out_lse[item] = M + logf(Z);
}

// ---------------------------------------------------------------------------
// plain VALU kernels (float32, or shapes outside the MFMA path)
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) score_generic(DecodeArgs a) {
  __shared__ float qs[256];
  __shared__ uint64_t red[4];
  const int tile = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int k = tile * 256 + t;
  const int D = a.d;
  const T* C = static_cast<const T*>(a.C) + size_t(h) * a.K * D;
  const T* q = static_cast<const T*>(a.qs);
  const float ci = k < a.K ? a.cinv[size_t(h) * a.K + k] : 0.0f;
  for (int b = 0; b < a.B; ++b) {
    for (int x = t; x < D; x += 256) qs[x] = load_elem(q, (size_t(b) * a.Hq + h) * D + x);
    __syncthreads();
    uint64_t key = 0;
    if (k < a.K) {
      float s = 0.0f;
      for (int x = 0; x < D; ++x) s = fmaf(qs[x], load_elem(C, size_t(k) * D + x), s);
      key = argmax_key(s * ci, uint32_t(k));
    }
    key = wave_max_u64(key);
    if (lane == 0) red[w] = key;
    __syncthreads();
    if (t == 0)
      a.keys[(size_t(h) * a.score_tiles + tile) * a.B + b] =
          umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
    __syncthreads();
  }
}

template <typename T>
__global__ void __launch_bounds__(256) attn_generic(DecodeArgs a) {
  const int item = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int split = item % a.S_max;
  const int bg = item / a.S_max;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv, D = a.d;
  const int n = a.kv_len[b];
  const int64_t st = a.kv_start[b];
  if (n < 0 || n > a.max_kv_len || st < 0 || st + n > a.kv_capacity) return;
  const int t_lo = split * a.split_tok;
  if (t_lo >= n) return;
  const int t_hi = min(n, t_lo + a.split_tok);
  const T* Kg = static_cast<const T*>(a.Kl) + g * a.kv_head_stride + st * a.kv_tok_stride;
  const T* Vg = static_cast<const T*>(a.Vl) + g * a.kv_head_stride + st * a.kv_tok_stride;
  const T* q = static_cast<const T*>(a.q);
  for (int hh = w; hh < G; hh += 4) {
    const int h = g * G + hh;
    float qv[4], acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane + 64 * j;
      qv[j] = x < D ? load_elem(q, (size_t(b) * a.Hq + h) * D + x) : 0.0f;
      acc[j] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    for (int tok = t_lo; tok < t_hi; ++tok) {
      const size_t off = size_t(tok) * a.kv_tok_stride;
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = lane + 64 * j;
        if (x < D) s = fmaf(qv[j], load_elem(Kg, off + x), s);
      }
      s = wave_sum(s) * a.scale2;
      const float mn = fmaxf(m, s);
      const float al = __builtin_amdgcn_exp2f(m - mn);
      const float p = __builtin_amdgcn_exp2f(s - mn);
      l = l * al + p;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = lane + 64 * j;
        const float v = x < D ? load_elem(Vg, off + x) : 0.0f;
        acc[j] = fmaf(p, v, acc[j] * al);
      }
      m = mn;
    }
    const size_t slot = (size_t(b) * a.Hq + h) * a.S_max + split;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane + 64 * j;
      if (x < D) a.part_a[slot * D + x] = acc[j] / l;
    }
    if (lane == 0) a.part_lse[slot] = (m + __log2f(l)) * ASM_LN2;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
  // the planner chose the path (and sized the workspace for it)
  if (a.n_waves > 0) return launch_decode_fast(a, s);
  const int n_attn = a.B * a.Hkv * a.S_max;
  if (dtype == 1) {
    hipLaunchKernelGGL(score_generic<float>, dim3(a.score_tiles, a.Hq), dim3(256), 0, s, a);
    if (n_attn > 0) hipLaunchKernelGGL(attn_generic<float>, dim3(n_attn), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(score_generic<uint16_t>, dim3(a.score_tiles, a.Hq), dim3(256), 0, s, a);
    if (n_attn > 0) hipLaunchKernelGGL(attn_generic<uint16_t>, dim3(n_attn), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(decode_combine_split, dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace asmk

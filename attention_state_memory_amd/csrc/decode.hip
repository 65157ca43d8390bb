// Decode step of attention-state memory on gfx950.
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Inferencia Online -- Recuperación (nearest
// centroid by cosine) and Fusión (merge the retrieved state with the query's
// attention over the non-prefix tokens by the online-softmax identity).
//
// One step is two launches on the caller's stream:
//   decode_main   a single grid holding two kinds of workgroups:
//                 * attention items (b, kv head g, token split): the G query
//                   heads of a GQA group attend one split of the sequence's
//                   local KV; scores come from MFMA (q rows x K^T), the
//                   value sum runs on the VALU in fp32; each item writes a
//                   partial state (a, lse) per query head;
//                 * scoring items (head h, 256-centroid tile): q . C^T on
//                   MFMA for all sequences, scaled by 1/|c|, reduced to one
//                   packed (score, index) key per (tile, sequence).
//   decode_combine one wave per (b, h): reduces the tile keys to the index,
//                 gathers the memory state, merges it with the split
//                 partials and writes out / out_lse / out_idx.
// float32 inputs, other head dims and other GQA group sizes run through the
// plain VALU kernels at the bottom of this file, which fill the same
// workspace and share decode_combine.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

// ---------------------------------------------------------------------------
// scoring: one 256-centroid tile of one head, all sequences
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void score_item(const DecodeArgs& a, int item, uint64_t* lk) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int h = item / a.score_tiles, tile = item % a.score_tiles;
  const uint16_t* Ch = static_cast<const uint16_t*>(a.C) + size_t(h) * a.K * D;
  const float* ci = a.cinv + size_t(h) * a.K;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  for (int q0 = 0; q0 < a.B; q0 += 32) {
    // B operand: query columns q0 + 16*nt + r16, d chunk 32*s + 8*grp.
    bf16x8 qb[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int b = q0 + 16 * nt + r16;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qb[nt][s] = as_bf16x8(b < a.B ? ld16(qp + (size_t(b) * a.Hq + h) * D + 32 * s + 8 * grp) : zero);
    }
    uint64_t best[2] = {0ull, 0ull};
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row0 = tile * 256 + w * 64 + rt * 16;
      if (row0 >= a.K) break;
      // A operand: centroid rows row0 + r16.
      const int row = row0 + r16;
      bf16x8 cb[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        cb[s] = as_bf16x8(row < a.K ? ld16(Ch + size_t(row) * D + 32 * s + 8 * grp) : zero);
      float cv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = row0 + 4 * grp + i;
        cv[i] = rr < a.K ? ci[rr] : 0.0f;
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cb[s], qb[nt][s], acc, 0, 0, 0);
        // acc[i] = score of centroid row0 + 4*grp + i against query column r16.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = row0 + 4 * grp + i;
          if (rr < a.K) best[nt] = umax64(best[nt], argmax_key(acc[i] * cv[i], uint32_t(rr)));
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      best[nt] = umax64(best[nt], shfl_xor_u64(best[nt], 16));
      best[nt] = umax64(best[nt], shfl_xor_u64(best[nt], 32));
    }
    if (grp == 0) {
      lk[w * 32 + r16] = best[0];
      lk[w * 32 + 16 + r16] = best[1];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      uint64_t k = lk[threadIdx.x];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) k = umax64(k, lk[ww * 32 + threadIdx.x]);
      const int b = q0 + threadIdx.x;
      if (b < a.B) a.keys[(size_t(h) * a.score_tiles + tile) * a.B + b] = k;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// local attention: one token split of one (sequence, kv head), G query heads
// ---------------------------------------------------------------------------
template <int D, int G>
struct AttnSmem {
  static constexpr int kP = 4 * 32 * G;            // per-wave probability tiles
  static constexpr int kC = 4 * G * (D + 2);       // per-wave (acc, m, l)
  static constexpr int kFloats = kP + kC;
};

template <int D, int G>
__device__ __forceinline__ void attn_item(const DecodeArgs& a, int item, float* smem) {
  constexpr int KS = D / 32;       // MFMA k-steps over the head dim
  constexpr int LPT = D / 8;       // lanes per token row in the value pass
  constexpr int TPI = 64 / LPT;    // token rows per wave-wide value load
  constexpr int NR = 32 / TPI;     // value rows per lane per 32-token tile
  constexpr int NG = (G + 3) / 4;  // lane groups that hold real head rows
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int split = item % a.S_max;
  const int bg = item / a.S_max;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int n = a.kv_len[b];
  const int64_t st = a.kv_start[b];
  if (n < 0 || n > a.max_kv_len || st < 0 || st + n > a.kv_capacity) return;
  const int t_lo = split * a.split_tok;
  if (t_lo >= n) return;
  const int t_hi = min(n, t_lo + a.split_tok);
  const int64_t ts = a.kv_tok_stride;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.Kl) + g * a.kv_head_stride + st * ts;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.Vl) + g * a.kv_head_stride + st * ts;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // A operand: head rows (r16 < G), d chunk 32*s + 8*grp.
  bf16x8 qa[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qa[s] = as_bf16x8(r16 < G ? ld16(qp + (size_t(b) * a.Hq + g * G + r16) * D + 32 * s + 8 * grp) : zero);

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;

  float* pl = smem + w * 32 * G;
  const int ntiles = (t_hi - t_lo + 31) >> 5;
  const int tsub = lane / LPT, dd0 = 8 * (lane % LPT);

  for (int tt = w; tt < ntiles; tt += 4) {
    const int t0 = t_lo + tt * 32;
    u32x4 kr[2][KS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tok = t0 + 16 * j + r16;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kr[j][s] = tok < t_hi ? ld16(Kg + size_t(tok) * ts + 32 * s + 8 * grp) : zero;
    }
    u32x4 vr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int tok = t0 + tsub + TPI * r;
      vr[r] = tok < t_hi ? ld16(Vg + size_t(tok) * ts + dd0) : zero;
    }
    f32x4 sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(kr[j][s]), sc[j], 0, 0, 0);
    }
    // sc[j][i]: head row 4*grp + i, token t0 + 16*j + r16 (base-2 logits below).
    const bool v0 = t0 + r16 < t_hi, v1 = t0 + 16 + r16 < t_hi;
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = v0 ? sc[0][i] * a.scale2 : -INFINITY;
      const float s1 = v1 ? sc[1][i] * a.scale2 : -INFINITY;
      float mt = fmaxf(s0, s1);
      mt = fmaxf(mt, shfl_xor_f(mt, 1));
      mt = fmaxf(mt, shfl_xor_f(mt, 2));
      mt = fmaxf(mt, shfl_xor_f(mt, 4));
      mt = fmaxf(mt, shfl_xor_f(mt, 8));
      const float mn = fmaxf(m_run[i], mt);
      alpha[i] = __builtin_amdgcn_exp2f(m_run[i] - mn);
      const float p0 = __builtin_amdgcn_exp2f(s0 - mn);
      const float p1 = __builtin_amdgcn_exp2f(s1 - mn);
      l_run[i] = l_run[i] * alpha[i] + p0 + p1;
      m_run[i] = mn;
      sc[0][i] = p0;
      sc[1][i] = p1;
    }
    if (grp < NG) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = 4 * grp + i;
        if (hh < G) {
          pl[r16 * G + hh] = sc[0][i];
          pl[(16 + r16) * G + hh] = sc[1][i];
        }
      }
    }
    float al[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) al[hh] = readlane_f(alpha[hh & 3], 16 * (hh >> 2));
    wave_lds_sync();
    bool rescale = false;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) rescale |= (al[hh] != 1.0f);
    if (rescale) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= al[hh];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int tl = tsub + TPI * r;
      float p[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) p[hh] = pl[tl * G + hh];
      float v[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[2 * c] = bf16_lo(vr[r][c]);
        v[2 * c + 1] = bf16_hi(vr[r][c]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p[hh], v[e], acc[hh][e]);
    }
    wave_lds_sync();
  }

  // wave totals
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    l_run[i] += shfl_xor_f(l_run[i], 1);
    l_run[i] += shfl_xor_f(l_run[i], 2);
    l_run[i] += shfl_xor_f(l_run[i], 4);
    l_run[i] += shfl_xor_f(l_run[i], 8);
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int m = LPT; m < 64; m <<= 1) acc[hh][e] += shfl_xor_f(acc[hh][e], m);

  float* cw = smem + AttnSmem<D, G>::kP;
  float* mine = cw + w * G * (D + 2);
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float mh = readlane_f(m_run[hh & 3], 16 * (hh >> 2));
    const float lh = readlane_f(l_run[hh & 3], 16 * (hh >> 2));
    if (lane == 0) {
      mine[hh * (D + 2) + D] = mh;
      mine[hh * (D + 2) + D + 1] = lh;
    }
    if (lane < LPT) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mine[hh * (D + 2) + dd0 + e] = acc[hh][e];
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < G * D; x += 256) {
    const int hh = x / D, dd = x % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, cw[(ww * G + hh) * (D + 2) + D]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float* c = cw + (ww * G + hh) * (D + 2);
      const float f = __builtin_amdgcn_exp2f(c[D] - M);  // waves without tokens: f = 0
      L += c[D + 1] * f;
      O += c[dd] * f;
    }
    const size_t slot = (size_t(b) * a.Hq + g * G + hh) * a.S_max + split;
    a.part_a[slot * D + dd] = O / L;
    if (dd == 0) a.part_lse[slot] = (M + __log2f(L)) * ASM_LN2;
  }
}

template <int D, int G>
__global__ void __launch_bounds__(256) decode_main_bf16(DecodeArgs a, int n_attn) {
  __shared__ float smem[AttnSmem<D, G>::kFloats];
  const int blk = blockIdx.x;
  if (blk < n_attn) {
    attn_item<D, G>(a, blk, smem);
  } else {
    score_item<D>(a, blk - n_attn, reinterpret_cast<uint64_t*>(smem));
  }
}

// ---------------------------------------------------------------------------
// combine: index, gather, merge
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_combine(DecodeArgs a) {
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
  const T* q = static_cast<const T*>(a.q);
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
bool decode_fast_path(int dtype, int d, int G) {
  return dtype == 0 && (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

template <int D, int G>
static void launch_main(const DecodeArgs& a, int n_attn, int n_score, hipStream_t s) {
  hipLaunchKernelGGL((decode_main_bf16<D, G>), dim3(n_attn + n_score), dim3(256), 0, s, a, n_attn);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int n_attn = a.B * a.Hkv * a.S_max;
  const int n_score = a.Hq * a.score_tiles;
  if (decode_fast_path(dtype, a.d, G)) {
    if (a.d == 128) {
      switch (G) {
        case 1: launch_main<128, 1>(a, n_attn, n_score, s); break;
        case 2: launch_main<128, 2>(a, n_attn, n_score, s); break;
        case 4: launch_main<128, 4>(a, n_attn, n_score, s); break;
        default: launch_main<128, 8>(a, n_attn, n_score, s); break;
      }
    } else {
      switch (G) {
        case 1: launch_main<64, 1>(a, n_attn, n_score, s); break;
        case 2: launch_main<64, 2>(a, n_attn, n_score, s); break;
        case 4: launch_main<64, 4>(a, n_attn, n_score, s); break;
        default: launch_main<64, 8>(a, n_attn, n_score, s); break;
      }
    }
  } else if (dtype == 1) {
    hipLaunchKernelGGL(score_generic<float>, dim3(a.score_tiles, a.Hq), dim3(256), 0, s, a);
    if (n_attn > 0) hipLaunchKernelGGL(attn_generic<float>, dim3(n_attn), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(score_generic<uint16_t>, dim3(a.score_tiles, a.Hq), dim3(256), 0, s, a);
    if (n_attn > 0) hipLaunchKernelGGL(attn_generic<uint16_t>, dim3(n_attn), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(decode_combine, dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace asmk

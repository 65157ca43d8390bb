// Decode step on MFMA (bf16, d in {64, 128}, GQA group G in {1, 2, 4, 8}).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Inferencia Online -- Recuperación (nearest
// centroid by cosine) and Fusión (merge the retrieved state with the query's
// attention over the non-prefix tokens by the online-softmax identity).
//
// The step is a stream over two kinds of 16 KB work units:
//   scoring unit   64 centroids of one query head against all B queries:
//                  q . C^T on MFMA (16x16x32 bf16), scaled by 1/|c|, packed
//                  into (score, index) keys, one key per (head, sequence,
//                  unit);
//   attention tile 32 local tokens of one (sequence, kv head): the G query
//                  heads of the group score the tile on MFMA, the online
//                  softmax runs on base-2 logits and the value sum on the
//                  fp32 VALU.
// decode_fast_main is a persistent grid of n_waves waves.  The scoring units
// and the attention tiles (in (sequence, kv head, token) order) are each cut
// into n_waves equal contiguous shares; every wave scores its share first,
// then attends its tiles, so ragged sequences cost no imbalance.  Each wave
// writes one partial state per (sequence, kv head) segment it touches.  decode_fast_combine (one wave per (b, h))
// reduces the keys to the index, gathers the memory state and merges it
// with the segment's partial states.
#include <atomic>

#include "common.hpp"
#include "hier_lookup.hpp"
#include "kernels.hpp"

namespace asmk {

// Issue the next tile's loads before consuming the current one.
constexpr bool kDecodePrefetch = true;

namespace {

__device__ __forceinline__ int64_t share_lo(int64_t w, int64_t total, int64_t W) {
  return w * total / W;
}
// Waves that take attention tiles: all of them, unless the scoring work is
// the larger part and the grid is capped, in which case the first waves
// attend and the rest score, in proportion to the two amounts of work.
__device__ __forceinline__ int64_t attention_waves(const DecodeArgs& a, int64_t W) {
  const int64_t SU = int64_t(a.Hq) * a.score_uph;
  const int64_t Umax = int64_t(a.B) * a.Hkv * ((int64_t(a.max_kv_len) + 31) / 32);
  if (SU + Umax <= W || Umax >= SU) return W;
  const int64_t A = W * Umax / (SU + Umax);
  return A < 1 ? 1 : A;
}
// the wave whose share holds unit x (inverse of share_lo)
__device__ __forceinline__ int64_t wave_of(int64_t x, int64_t total, int64_t W) {
  return ((x + 1) * W - 1) / total;
}

__device__ __forceinline__ bool seq_valid(const DecodeArgs& a, int b) {
  const int n = a.kv_len[b];
  const int64_t st = a.kv_start[b];
  return n >= 0 && n <= a.max_kv_len && st >= 0 && st + n <= a.kv_capacity;
}

// ---------------------------------------------------------------------------
// scoring units: centroids [64*j, 64*j + 64) of head h against all sequences
// ---------------------------------------------------------------------------
// A unit is consumed as two halves of 32 centroids.  What one half reads
// besides the queries: 32 centroid rows and their inverse norms, with a
// single round trip.  Rows past K read as zeros through the buffer bounds; a
// half index past the wave's share loads nothing.
template <int D>
struct ScoreHalf {
  static constexpr int KS = D / 32;
  u32x4 c[2][KS];  // A operand: centroid rows of two 16-row tiles
  float cv[2][4];  // inverse norms of rows 4*grp + i of each tile
};

// half v covers centroids 32*(v % (2*uph)) .. +32 of head v / (2*uph)
template <int D>
__device__ __forceinline__ void load_half(ScoreHalf<D>& t, const DecodeArgs& a, int v, int SV) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const bool live = v < SV;
  const int h = live ? v / (2 * a.uph) : 0;
  const int c0 = live ? (v - h * 2 * a.uph) * 32 : 0;
  const uint32_t cbytes = uint32_t(a.K) * D * 2;
  const auto rc = make_rsrc(static_cast<const uint16_t*>(a.C) + size_t(h) * a.K * D, cbytes);
  const auto ri = make_rsrc(a.cinv + size_t(h) * a.K, uint32_t(a.K) * 4);
  const int cdead = live ? 0 : int(cbytes);
  const int idead = live ? 0 : a.K * 4;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = c0 + rt * 16 + r16;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.c[rt][s] = buf16(rc, (row * D + 32 * s + 8 * grp) * 2 + cdead, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.cv[rt][i] = buf_f32(ri, (c0 + rt * 16 + 4 * grp + i) * 4 + idead, 0);
  }
}

// B operand: query columns q0 + 16*nt + r16 of head h (past B: zeros).
template <int D>
__device__ __forceinline__ void load_queries(u32x4 (&qb)[2][D / 32], const DecodeArgs& a, int h,
                                             int q0) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const auto rq = make_rsrc(a.qs, uint32_t(a.B) * a.Hq * D * 2);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int b = q0 + 16 * nt + r16;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[nt][s] = buf16(rq, ((b * a.Hq + h) * D + 32 * s + 8 * grp) * 2, 0);
  }
}

template <int D>
__device__ __forceinline__ void consume_half(const ScoreHalf<D>& t, const u32x4 (&qb)[2][D / 32],
                                             const DecodeArgs& a, int c0, uint64_t (&best)[2]) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row0 = c0 + rt * 16;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.c[rt][s]), as_bf16x8(qb[nt][s]), acc,
                                                      0, 0, 0);
      // acc[i]: centroid row0 + 4*grp + i against query column q0 + 16*nt + r16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = row0 + 4 * grp + i;
        const uint64_t key = argmax_key(acc[i] * t.cv[rt][i], uint32_t(rr));
        best[nt] = umax64(best[nt], rr < a.K ? key : 0ull);
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_keys(const DecodeArgs& a, int h, int j, int q0,
                                           uint64_t (&best)[2]) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    best[nt] = umax64(best[nt], shfl_xor_u64(best[nt], 16));
    best[nt] = umax64(best[nt], shfl_xor_u64(best[nt], 32));
    const int b = q0 + 16 * nt + r16;
    if (grp == 0 && b < a.B) a.keys[(size_t(h) * a.B + b) * a.uph + j] = best[nt];
    best[nt] = 0ull;
  }
}

// Units [lo, hi) of this wave.  Units of one head are contiguous; per head
// (and per slice of 32 sequences) the queries are loaded once and the loop
// over half units keeps two halves in flight: the next half's loads are
// issued before the current one is consumed, and are never skipped, so the
// compiler waits for exactly one half's loads.
template <int D>
__device__ __forceinline__ void score_range(const DecodeArgs& a, int lo, int hi, int SU) {
  const int SV = 2 * SU;
  int u0 = lo;
  while (u0 < hi) {
    const int h = u0 / a.uph;
    const int u1 = min(hi, (h + 1) * a.uph);
    for (int q0 = 0; q0 < a.B; q0 += 32) {
      u32x4 qb[2][D / 32];
      load_queries<D>(qb, a, h, q0);
      uint64_t best[2] = {0ull, 0ull};
      ScoreHalf<D> ta, tb;
      load_half<D>(ta, a, 2 * u0, SV);
      for (int u = u0; u < u1; ++u) {
        const int j = u - h * a.uph;
        load_half<D>(tb, a, 2 * u + 1, SV);
        consume_half<D>(ta, qb, a, 64 * j, best);
        load_half<D>(ta, a, u + 1 < u1 ? 2 * u + 2 : SV, SV);
        consume_half<D>(tb, qb, a, 64 * j + 32, best);
        store_keys<D>(a, h, j, q0, best);
      }
    }
    u0 = u1;
  }
}

// ---------------------------------------------------------------------------
// attention: tiles [j0, j1) of segment (b, g), one wave, one partial state
// ---------------------------------------------------------------------------
template <int D, int G>
struct Tile {
  static constexpr int KS = D / 32;     // MFMA k-steps over the head dim
  static constexpr int LPT = D / 8;     // lanes per token row in the value pass
  static constexpr int TPI = 64 / LPT;  // token rows per wave-wide value load
  static constexpr int NR = 32 / TPI;   // value rows per lane per tile
  static constexpr int NG = (G + 3) / 4;
  u32x4 k[2][KS];
  u32x4 v[NR];
};

// Per-lane byte offsets of one tile relative to the tile's first token; the
// tile start enters as the scalar offset.  Tokens past the segment end read
// as zeros (buffer bounds): their scores are masked and their weights are 0.
template <int D, int G>
struct TileOffsets {
  int k[2];
  int v[Tile<D, G>::NR];
  __device__ __forceinline__ TileOffsets(int64_t ts) {
    using T = Tile<D, G>;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, grp = lane >> 4;
    const int tsub = lane / T::LPT, dd0 = 8 * (lane % T::LPT);
    const int t32 = int(ts);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) k[jj] = ((16 * jj + r16) * t32 + 8 * grp) * 2;
#pragma unroll
    for (int r = 0; r < T::NR; ++r) v[r] = ((tsub + T::TPI * r) * t32 + dd0) * 2;
  }
};

// The tile start is added to the per-lane offsets (not passed as the scalar
// offset) so that the buffer bounds check covers it; a tile start at or past
// the segment end loads zeros without touching memory.
template <int D, int G>
__device__ __forceinline__ void load_tile(Tile<D, G>& t, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, const TileOffsets<D, G>& o,
                                          int start) {
  using T = Tile<D, G>;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int s = 0; s < T::KS; ++s) t.k[jj][s] = buf16(rk, o.k[jj] + start + 64 * s, 0);
#pragma unroll
  for (int r = 0; r < T::NR; ++r) t.v[r] = buf16(rv, o.v[r] + start, 0);
}

template <int D, int G>
struct Running {
  float m[4], l[4];  // per head row 4*grp + i, base-2
  float acc[G][8];   // value sums, dims 8*(lane % LPT) .. +8, token subset lane / LPT
};

template <int D, int G>
__device__ __forceinline__ void consume_tile(const Tile<D, G>& t, Running<D, G>& st,
                                             const bf16x8 (&qa)[D / 32], float scale2,
                                             int nvalid, float* pl) {
  using T = Tile<D, G>;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int tsub = lane / T::LPT;
  f32x4 sc[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    sc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
      sc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(t.k[jj][s]), sc[jj], 0, 0, 0);
  }
  // sc[jj][i]: head row 4*grp + i, token 16*jj + r16 of the tile
  const bool v0 = r16 < nvalid, v1 = 16 + r16 < nvalid;
  float alpha[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s0 = v0 ? sc[0][i] * scale2 : -INFINITY;
    const float s1 = v1 ? sc[1][i] * scale2 : -INFINITY;
    const float mt = row16_max(fmaxf(s0, s1));
    const float mn = fmaxf(st.m[i], mt);  // finite: every tile holds a valid token
    alpha[i] = __builtin_amdgcn_exp2f(st.m[i] - mn);
    const float p0 = __builtin_amdgcn_exp2f(s0 - mn);
    const float p1 = __builtin_amdgcn_exp2f(s1 - mn);
    st.l[i] = st.l[i] * alpha[i] + p0 + p1;
    st.m[i] = mn;
    sc[0][i] = p0;
    sc[1][i] = p1;
  }
  if (grp < T::NG) {
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
      for (int e = 0; e < 8; ++e) st.acc[hh][e] *= al[hh];
  }
#pragma unroll
  for (int r = 0; r < T::NR; ++r) {
    const int tl = tsub + T::TPI * r;
    float p[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) p[hh] = pl[tl * G + hh];
    float v[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[2 * c] = bf16_lo(t.v[r][c]);
      v[2 * c + 1] = bf16_hi(t.v[r][c]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[hh][e] = fmaf(p[hh], v[e], st.acc[hh][e]);
  }
  wave_lds_sync();
}

template <int D, int G, bool kPrefetch>
__device__ __forceinline__ void attn_piece(const DecodeArgs& a, int b, int g, int j0, int j1,
                                           int64_t piece, float* pl) {
  using T = Tile<D, G>;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int n = __builtin_amdgcn_readfirstlane(a.kv_len[b]);
  const int64_t st0 = __builtin_amdgcn_readfirstlane(a.kv_start[b]);
  const int64_t ts = a.kv_tok_stride;
  const uint32_t seg_bytes = uint32_t(n) * uint32_t(ts) * 2u;
  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.Kl) + g * a.kv_head_stride + st0 * ts, seg_bytes);
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.Vl) + g * a.kv_head_stride + st0 * ts, seg_bytes);
  const TileOffsets<D, G> off(ts);
  const int tile_bytes = 32 * int(ts) * 2;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  bf16x8 qa[T::KS];  // A operand: head rows r16 < G
#pragma unroll
  for (int s = 0; s < T::KS; ++s)
    qa[s] = as_bf16x8(r16 < G ? ld16(qp + (size_t(b) * a.Hq + g * G + r16) * D + 32 * s + 8 * grp) : zero);

  Running<D, G> st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.m[i] = -INFINITY;
    st.l[i] = 0.0f;
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[hh][e] = 0.0f;

  if constexpr (kPrefetch) {
    // Two register tiles in flight.  The prefetch is never skipped (a
    // finished piece prefetches from past the segment end, which loads
    // nothing), so the compiler can wait for exactly one tile's loads.
    const int end_off = int(seg_bytes);
    Tile<D, G> ta, tb;
    load_tile<D, G>(ta, rk, rv, off, j0 * tile_bytes);
    for (int j = j0; j < j1; j += 2) {
      load_tile<D, G>(tb, rk, rv, off, j + 1 < j1 ? (j + 1) * tile_bytes : end_off);
      consume_tile<D, G>(ta, st, qa, a.scale2, min(32, n - 32 * j), pl);
      if (j + 1 >= j1) break;
      load_tile<D, G>(ta, rk, rv, off, j + 2 < j1 ? (j + 2) * tile_bytes : end_off);
      consume_tile<D, G>(tb, st, qa, a.scale2, min(32, n - 32 * (j + 1)), pl);
    }
  } else {
    for (int j = j0; j < j1; ++j) {
      Tile<D, G> t;
      load_tile<D, G>(t, rk, rv, off, j * tile_bytes);
      consume_tile<D, G>(t, st, qa, a.scale2, min(32, n - 32 * j), pl);
    }
  }

  // wave totals: l over the 16 token lanes, acc over the token subsets
#pragma unroll
  for (int i = 0; i < 4; ++i) st.l[i] = row16_sum(st.l[i]);
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int m = T::LPT; m < 64; m <<= 1) st.acc[hh][e] += shfl_xor_f(st.acc[hh][e], m);
  const int dd0 = 8 * (lane % T::LPT);
  float* pa = a.part_a + size_t(piece) * G * D;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float mh = readlane_f(st.m[hh & 3], 16 * (hh >> 2));
    const float lh = readlane_f(st.l[hh & 3], 16 * (hh >> 2));
    const float inv = 1.0f / lh;
    if (lane < T::LPT) {
      f32x4 o0, o1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = st.acc[hh][e] * inv;
        o1[e] = st.acc[hh][4 + e] * inv;
      }
      *reinterpret_cast<f32x4*>(pa + hh * D + dd0) = o0;
      *reinterpret_cast<f32x4*>(pa + hh * D + dd0 + 4) = o1;
    }
    if (lane == 0) a.part_lse[size_t(piece) * G + hh] = (mh + __log2f(lh)) * ASM_LN2;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// One workgroup (block index blk) of the main grid.
template <int D, int G, bool kPrefetch>
__device__ __forceinline__ void main_block(const DecodeArgs& a, int blk) {
  __shared__ int32_t tp[kFastMaxBatch + 1];
  __shared__ int32_t wsum[4];
  __shared__ float pls[4 * 32 * G];
  // the wave index is uniform across the wave; telling the compiler keeps the
  // work-share arithmetic and the buffer resources in scalar registers
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int64_t gw = int64_t(blk) * 4 + w;
  const int64_t W = a.n_waves;
  const int64_t SU = int64_t(a.Hq) * a.score_uph;

  // The lengths of the first 256 sequences are loaded now and scanned after
  // the scoring share, which does not need them.
  const int v_first = (int(threadIdx.x) < a.B && seq_valid(a, threadIdx.x)) ? (a.kv_len[threadIdx.x] + 31) >> 5 : 0;

  // Scoring share first: every wave scores at the same time, so the table
  // streams with the whole grid's memory parallelism.  When the grid has a
  // wave for every unit (small steps, which are latency-bound), the scoring
  // units go to the last SU waves and the attention tiles to the first ones,
  // so that no wave does both one after the other.
  const int64_t Umax = int64_t(a.B) * a.Hkv * ((int64_t(a.max_kv_len) + 31) / 32);
  const int64_t A = attention_waves(a, W);
  if (SU + Umax <= W) {
    const int64_t su = gw - (W - SU);
    if (su >= 0) score_range<D>(a, int(su), int(su + 1), int(SU));
  } else if (A < W) {
    const int64_t gs = gw - A;  // scoring waves A .. W-1
    if (gs >= 0) score_range<D>(a, int(share_lo(gs, SU, W - A)), int(share_lo(gs + 1, SU, W - A)), int(SU));
  } else {
    score_range<D>(a, int(share_lo(gw, SU, W)), int(share_lo(gw + 1, SU, W)), int(SU));
  }

  // tiles per kv head of every sequence, exclusive prefix over sequences
  int carry = 0;
  for (int base = 0; base < a.B; base += 256) {
    const int b = base + threadIdx.x;
    const int v = base == 0 ? v_first : (b < a.B && seq_valid(a, b)) ? (a.kv_len[b] + 31) >> 5 : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int before = carry;
    for (int ww = 0; ww < w; ++ww) before += wsum[ww];
    if (b < a.B) tp[b] = before + x - v;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) tp[a.B] = carry;
  __syncthreads();
  if (blk == 0)
    for (int b = threadIdx.x; b <= a.B; b += 256) a.tile_prefix[b] = tp[b];
  const int64_t U = int64_t(__builtin_amdgcn_readfirstlane(tp[a.B])) * a.Hkv;

  // Attention shares go to the first min(W, U) waves only, so that every
  // share holds at least one tile and the pieces of a segment sit at
  // consecutive indices.
  float* pl = pls + w * 32 * G;
  const int64_t Wa = min(A, U);
  int64_t t = gw < Wa ? share_lo(gw, U, Wa) : 0;
  const int64_t t_end = gw < Wa ? share_lo(gw + 1, U, Wa) : 0;
  while (t < t_end) {
    // LDS reads land in vector registers; readfirstlane marks the (wave-
    // uniform) values as scalars so the buffer resources built from them stay
    // in SGPRs (otherwise every buffer load becomes a waterfall loop).
    int blo = 0, bhi = a.B;  // tp[blo]*Hkv <= t < tp[bhi]*Hkv
    while (bhi - blo > 1) {
      const int mid = (blo + bhi) >> 1;
      if (int64_t(__builtin_amdgcn_readfirstlane(tp[mid])) * a.Hkv <= t) blo = mid; else bhi = mid;
    }
    const int b = blo;
    const int tb0 = __builtin_amdgcn_readfirstlane(tp[b]);
    const int nt = __builtin_amdgcn_readfirstlane(tp[b + 1]) - tb0;
    const int64_t off = t - int64_t(tb0) * a.Hkv;
    const int g = int(off / nt), j0 = int(off % nt);
    const int cnt = int(min<int64_t>(nt - j0, t_end - t));
    attn_piece<D, G, kPrefetch>(a, b, g, j0, j0 + cnt, gw + int64_t(b) * a.Hkv + g, pl);
    t += cnt;
  }
}

template <int D, int G, bool kPrefetch>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kPrefetch ? 2 : 3)))
decode_fast_main(DecodeArgs a) {
  main_block<D, G, kPrefetch>(a, int(blockIdx.x));
}

// The two-level lookup fused into the main grid: the first lookup_blocks
// workgroups run the lookup (one per sequence, head and probe rank) and the
// rest run the attention shares (scoring off).  The two roles share no
// data inside the kernel -- the lookup writes the unit keys that the combine
// reduces -- so at small batch they run side by side instead of one launch
// after the other.
template <int D, int G, bool kPrefetch>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kPrefetch ? 2 : 3)))
decode_fast_main_hier(DecodeArgs a, HierArgs h, int lookup_blocks) {
  if (int(blockIdx.x) < lookup_blocks)
    hier_lookup_block<D>(h, int(blockIdx.x));
  else
    main_block<D, G, kPrefetch>(a, int(blockIdx.x) - lookup_blocks);
}

// One wave per (b, h): index from the unit keys, gather of the memory
// state, merge with the partial states of segment (b, h / G).  The loads are
// arranged in two dependent rounds: (1) sequence bounds, tile prefix, keys;
// (2) the gathered memory state, the piece normalisers and the first 16
// piece rows (rows past the last piece read as zeros through the buffer
// bounds); later pieces, if any, follow 16 rows at a time.
template <int G>
__global__ void __launch_bounds__(256) decode_fast_combine(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values stay in scalar registers (so the loads of the
  // sequence bounds are scalar and the piece buffer resource needs no
  // per-lane waterfall loop)
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= a.B * a.Hq) return;
  const int b = item / a.Hq, h = item % a.Hq;
  const int g = h / G, hh = h % G;
  const int D = a.d;  // 64 or 128: lane owns dims 2*lane, 2*lane + 1
  // round 1
  const int tpb = a.tile_prefix[b], tpb1 = a.tile_prefix[b + 1], tpB = a.tile_prefix[a.B];
  const bool valid = seq_valid(a, b);
  const uint64_t* kk = a.keys + (size_t(h) * a.B + b) * a.uph;
  uint64_t best = 0;
  for (int u = lane; u < a.uph; u += 64) best = umax64(best, kk[u]);
  const int nt = tpb1 - tpb;
  int64_t p0 = 0, np = 0;  // pieces of segment (b, g)
  if (nt > 0) {
    const int64_t total = int64_t(tpB) * a.Hkv;
    const int64_t W = min<int64_t>(attention_waves(a, a.n_waves), total);
    const int64_t first = int64_t(tpb) * a.Hkv + int64_t(g) * nt;
    const int64_t seg = int64_t(b) * a.Hkv + g;
    p0 = wave_of(first, total, W) + seg;
    np = wave_of(first + nt - 1, total, W) + seg - p0 + 1;
  }
  best = wave_max_u64(best);
  const uint32_t k = __builtin_amdgcn_readfirstlane(key_index(best));
  if (lane == 0 && a.out_idx) a.out_idx[item] = int32_t(k);
  float* o = a.out + size_t(item) * D;
  const int dd = 2 * lane;
  if (!valid || k >= uint32_t(a.K)) {
    if (dd < D) *reinterpret_cast<float2*>(o + dd) = make_float2(NAN, NAN);
    if (lane == 0 && a.out_lse) a.out_lse[item] = NAN;
    return;
  }
  // round 2
  const float lm = a.LSEbar[size_t(h) * a.K + k];
  const float2 am = dd < D ? *reinterpret_cast<const float2*>(a.Abar + (size_t(h) * a.K + k) * D + dd)
                           : make_float2(0.f, 0.f);
  const float* pa0 = a.part_a + (p0 * G + hh) * D;
  const auto rp = make_rsrc(pa0, np > 0 ? uint32_t(((np - 1) * G + 1) * D * 4) : 0u);
  // the first 64 piece normalisers and the first 16 piece rows load with the
  // memory state (rows past the last piece read as zeros)
  const float lc0 = lane < np ? a.part_lse[(p0 + lane) * G + hh] : -INFINITY;
  u32x2 r0[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    r0[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                          rp, int((i * G * D + dd) * 4), 0, 0));
  float M = fmaxf(lm, lc0);
  for (int64_t c = 64 + lane; c < np; c += 64) M = fmaxf(M, a.part_lse[(p0 + c) * G + hh]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor_f(M, m));
  if (M == -INFINITY) {
    if (dd < D) *reinterpret_cast<float2*>(o + dd) = make_float2(0.f, 0.f);
    if (lane == 0 && a.out_lse) a.out_lse[item] = -INFINITY;
    return;
  }
  const float wm = lm == -INFINITY ? 0.0f : expf(lm - M);
  float v0 = wm > 0.0f ? wm * am.x : 0.0f, v1 = wm > 0.0f ? wm * am.y : 0.0f;
  float zsum = 0.0f;
  for (int64_t c64 = 0; c64 < np; c64 += 64) {
    const float lc = c64 == 0 ? lc0
                   : (c64 + lane < np ? a.part_lse[(p0 + c64 + lane) * G + hh] : -INFINITY);
    const float wc = lc == -INFINITY ? 0.0f : expf(lc - M);
    zsum += wc;
    const int64_t cend = min<int64_t>(np, c64 + 64);
    for (int64_t c = c64; c < cend; c += 16) {
      u32x2 r[16];
      if (c == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) r[i] = r0[i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          r[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                               rp, int(((c + i) * G * D + dd) * 4), 0, 0));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float wi = readlane_f(wc, int(c - c64) + i);
        v0 = fmaf(wi, __uint_as_float(r[i][0]), v0);
        v1 = fmaf(wi, __uint_as_float(r[i][1]), v1);
      }
    }
  }
  const float Z = wm + wave_sum(zsum);
  const float inv = 1.0f / Z;
  if (dd < D) *reinterpret_cast<float2*>(o + dd) = make_float2(v0 * inv, v1 * inv);
  if (lane == 0 && a.out_lse) a.out_lse[item] = M + logf(Z);
}

// ---------------------------------------------------------------------------
bool decode_fast_path(int dtype, int d, int G, int64_t kv_tok_stride, int max_kv_len) {
  // buffer offsets are 32-bit: one sequence's KV rows must span < 2 GiB
  const bool fits = int64_t(max_kv_len + 32) * kv_tok_stride * 2 < (int64_t(1) << 31);
  return dtype == 0 && (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8) && fits;
}

template <int D, int G>
static void launch_fast_hier(const DecodeArgs& a, const HierArgs& h, hipStream_t s) {
  const int lookup_blocks = a.B * a.Hq * h.p;
  hipLaunchKernelGGL((decode_fast_main_hier<D, G, kDecodePrefetch>), dim3(unsigned(lookup_blocks + a.n_waves / 4)),
                     dim3(256), 0, s, a, h, lookup_blocks);
  hipLaunchKernelGGL((decode_fast_combine<G>), dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
}

template <int D, int G>
static void launch_fast(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_fast_main<D, G, kDecodePrefetch>), dim3(a.n_waves / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL((decode_fast_combine<G>), dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
}

template <int D, int G>
static int occupancy_waves() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_fast_main<D, G, kDecodePrefetch>,
                                                   256, 0) != hipSuccess || blocks < 1)
    blocks = 1;
  return 4 * blocks;
}

int decode_fast_waves_per_cu(int d, int G) {
  // Computed once per (d, G); host threads may race to fill an entry, but
  // they store the same value and the accesses are atomic.
  static std::atomic<int> cache[2][4];
  const int di = d == 128 ? 0 : 1;
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  int cached = cache[di][gi].load(std::memory_order_relaxed);
  if (cached == 0) {
    int v = 4;
    if (d == 128) {
      v = G == 1 ? occupancy_waves<128, 1>() : G == 2 ? occupancy_waves<128, 2>()
        : G == 4 ? occupancy_waves<128, 4>() : occupancy_waves<128, 8>();
    } else {
      v = G == 1 ? occupancy_waves<64, 1>() : G == 2 ? occupancy_waves<64, 2>()
        : G == 4 ? occupancy_waves<64, 4>() : occupancy_waves<64, 8>();
    }
    cache[di][gi].store(v, std::memory_order_relaxed);
    cached = v;
  }
  return cached;
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.d == 128) {
    switch (G) {
      case 1: launch_fast<128, 1>(a, s); break;
      case 2: launch_fast<128, 2>(a, s); break;
      case 4: launch_fast<128, 4>(a, s); break;
      default: launch_fast<128, 8>(a, s); break;
    }
  } else {
    switch (G) {
      case 1: launch_fast<64, 1>(a, s); break;
      case 2: launch_fast<64, 2>(a, s); break;
      case 4: launch_fast<64, 4>(a, s); break;
      default: launch_fast<64, 8>(a, s); break;
    }
  }
  return hipGetLastError();
}

bool hier_fast_path(int dtype, int d) { return dtype == 0 && (d == 64 || d == 128); }

hipError_t launch_decode_hier(const DecodeArgs& a, const HierArgs& h, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.d == 128) {
    switch (G) {
      case 1: launch_fast_hier<128, 1>(a, h, s); break;
      case 2: launch_fast_hier<128, 2>(a, h, s); break;
      case 4: launch_fast_hier<128, 4>(a, h, s); break;
      default: launch_fast_hier<128, 8>(a, h, s); break;
    }
  } else {
    switch (G) {
      case 1: launch_fast_hier<64, 1>(a, h, s); break;
      case 2: launch_fast_hier<64, 2>(a, h, s); break;
      case 4: launch_fast_hier<64, 4>(a, h, s); break;
      default: launch_fast_hier<64, 8>(a, h, s); break;
    }
  }
  return hipGetLastError();
}

}  // namespace asmk

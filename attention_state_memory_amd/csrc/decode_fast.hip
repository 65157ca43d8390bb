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
// decode_fast_main is a persistent grid of 8-wave workgroups (two waves per
// SIMD).  Waves w and w + 4 of a workgroup form a pair, and every pair gets
// the same pool: its share of the scoring units followed by its share of the
// tiles (in (sequence, kv head, token) order), so every compute unit streams
// the same bytes.  The pair's first wave takes items from the front of the
// pool and the second from the back, each claiming the next one from a
// counter in LDS, so the table and the local KV stream side by side and the
// wave the SIMD serves first (which streams well ahead of its sibling) does
// more of the pool.  Every wave writes one partial state per (sequence, kv
// head) segment of its pool's tiles (an empty one where it attended no
// tile).  decode_fast_combine (one wave per (b, h)) reduces the keys to the
// index, gathers the memory state and merges it with the segment's partial
// states.
#include <atomic>

#include "common.hpp"
#include "hier_lookup.hpp"
#include "kernels.hpp"

namespace asmk {


namespace {

__device__ __forceinline__ int64_t share_lo(int64_t w, int64_t total, int64_t W) {
  return w * total / W;
}
// How the W waves of the grid divide the step, given U attention tiles and SU
// scoring units (both known once the lengths are scanned).  The main kernel
// and the combine evaluate it on the same integers, so they agree on where
// every partial state lives.
//   disjoint  the grid has a wave for every unit (small, latency-bound
//             steps): one unit per wave, attention tiles on waves [0, U),
//             scoring units on waves [W - SU, W); ranks are waves;
//   mixed     (at least 4 tiles per pair) every wave pair p < P = W / 2 gets
//             the same mix: scoring units
//             [p SU / P, (p+1) SU / P) and, for the first Wa = min(P, U)
//             pairs, tiles [p U / Wa, (p+1) U / Wa).  The memory system
//             serves every compute unit about equally, so equal bytes per
//             pair (four pairs per compute unit) make the waves finish
//             together.  Ranks are pairs.
//   scarce    (fewer than 4 tiles per pair) the tiles and then the scoring
//             units, as one sequence of SU + U items, cut into P equal
//             contiguous ranges, one per pair, so that the tiles sit on
//             fewer pairs (a segment's partial states stay few) while every
//             pair still gets the same work.
// Tile x lives at rank wave_of(x, tot, Wt).
struct Roles {
  int64_t Wa;       // ranks that hold tiles
  bool disjoint;
  bool scarce;      // the contiguous layout for few tiles
  int64_t tot, Wt;  // tile x -> rank wave_of(x, tot, Wt)
};
__device__ __forceinline__ Roles plan_roles(const DecodeArgs& a, int64_t W, int64_t U) {
  const int64_t SU = int64_t(a.Hq) * a.score_uph;
  if (SU + U <= W) return {U, true, false, U, U};
  const int64_t P = W / 2;
  if (U < 4 * P) {
    const int64_t T = SU + U;
    return {U > 0 ? ((U * P - 1) / T) + 1 : 0, false, true, T, P};
  }
  const int64_t Wa = min(P, U);
  return {Wa, false, false, U, Wa};
}
// Partial-state slot of rank r's piece of segment seg: one per rank
// (disjoint) or one per wave of the pair (member m).  The slots of one
// segment are consecutive.
__device__ __forceinline__ int64_t piece_slot(bool disjoint, int64_t r, int64_t seg, int m) {
  return disjoint ? r + seg : 2 * (r + seg) + m;
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
// single round trip.  The half's first row moves the base of its buffer
// resources (scalar arithmetic), so the per-lane offsets are loop-invariant;
// rows past K read as zeros through the buffer bounds, and a half index past
// the wave's share loads nothing.
template <int D>
struct ScoreHalf {
  static constexpr int KS = D / 32;
  u32x4 c[2][KS];  // A operand: centroid rows of two 16-row tiles
  f32x4 cv[2];     // inverse norms of rows 4*grp .. 4*grp + 3 of each tile
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
  // K * D * 2 < 2^31 on this path; the last unit's second half can start at
  // or past K (then it reads nothing)
  const int rows_left = live && a.K > c0 ? a.K - c0 : 0;
  const char* cb = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.C) + (size_t(h) * a.K + c0) * D));
  const float* ib = uniform_ptr(a.cinv + size_t(h) * a.K + c0);
  const auto rc = make_rsrc(cb, uint32_t(rows_left) * D * 2);
  const auto ri = make_rsrc(ib, uint32_t(rows_left) * 4);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int s = 0; s < KS; ++s) t.c[rt][s] = buf16_nt(rc, ((rt * 16 + r16) * D + 8 * grp) * 2 + 64 * s, 0);
    t.cv[rt] = __builtin_bit_cast(f32x4, buf16_nt(ri, (rt * 16 + 4 * grp) * 4, 0));
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

// ---------------------------------------------------------------------------
// pools of a wave pair
// ---------------------------------------------------------------------------
// Units [lo, hi) shared by the two waves of a pair: member 0 takes them from
// the front, member 1 from the back.  A claim adds one to the pair's counter
// in LDS and succeeds while the counter was below the pool size, so the two
// ends never cross and every unit is taken by exactly one wave.  A wave that
// the SIMD serves faster simply claims more of the pool.
// A pool holds n items: its scoring units first (items [0, nsu), units
// su_lo ..), then its attention tiles (item nsu + i is tile t_lo + i).
struct PairPool {
  int32_t* ctr;   // in LDS, zero before the first claim
  int64_t n, nsu, su_lo, t_lo;
  int m;          // 0: front, 1: back
  int64_t taken;  // items this wave has taken
};
__device__ __forceinline__ int64_t claim(PairPool& p) {
  int c = 0;
  if ((threadIdx.x & 63) == 0) c = atomicAdd(p.ctr, 1);
  c = __builtin_amdgcn_readfirstlane(c);
  if (c >= p.n) return -1;
  const int64_t v = p.m == 0 ? p.taken : p.n - 1 - p.taken;
  ++p.taken;
  return v;
}
__device__ __forceinline__ bool pool_unit(const PairPool& p, int64_t v) { return v >= 0 && v < p.nsu; }
__device__ __forceinline__ int64_t pool_tile(const PairPool& p, int64_t v) {
  return v >= p.nsu ? p.t_lo + (v - p.nsu) : -1;
}

// One unit for all sequences, 32 at a time (batches above 32 sequences).
template <int D>
__device__ __forceinline__ void score_unit(const DecodeArgs& a, int64_t u, int SV) {
  const int h = int(u / a.uph), j = int(u - int64_t(h) * a.uph);
  for (int q0 = 0; q0 < a.B; q0 += 32) {
    u32x4 qb[2][D / 32];
    load_queries<D>(qb, a, h, q0);
    uint64_t best[2] = {0ull, 0ull};
    ScoreHalf<D> t0, t1;
    load_half<D>(t0, a, int(2 * u), SV);
    load_half<D>(t1, a, int(2 * u + 1), SV);
    consume_half<D>(t0, qb, a, 64 * j, best);
    consume_half<D>(t1, qb, a, 64 * j + 32, best);
    store_keys<D>(a, h, j, q0, best);
  }
}

// One unit in the direct layout's gathering steps (at most 8 sequences): its
// keys, and for every sequence the state (a row, lse) of the unit's best
// entry, copied to the unit's candidate slot, so that the merge finds the
// winner's state in the same round as the keys.  (Every unit holds a row
// below K, so its best key names an entry; an entry index past K is skipped
// all the same.)
template <int D>
__device__ __forceinline__ void score_unit_gather(const DecodeArgs& a, int64_t u, int SV) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int h = int(u / a.uph), j = int(u - int64_t(h) * a.uph);
  u32x4 qb[2][D / 32];
  load_queries<D>(qb, a, h, 0);
  uint64_t best[2] = {0ull, 0ull};
  ScoreHalf<D> t0, t1;
  load_half<D>(t0, a, int(2 * u), SV);
  load_half<D>(t1, a, int(2 * u + 1), SV);
  consume_half<D>(t0, qb, a, 64 * j, best);
  consume_half<D>(t1, qb, a, 64 * j + 32, best);
  // lane (r16, *) now reduces sequence r16's key (at most 8 sequences: the
  // first column tile only)
  uint64_t kq = best[0];
  kq = umax64(kq, shfl_xor_u64(kq, 16));
  kq = umax64(kq, shfl_xor_u64(kq, 32));
  if (grp == 0 && r16 < a.B) a.keys[(size_t(h) * a.B + r16) * a.uph + j] = kq;
  // the best entries' states: all loads first (sequences past B repeat the
  // last one), then the stores
  const int dd = 2 * lane;
  float2 va[8];
  float vl[8];
  uint32_t ev[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int bb = b < a.B ? b : a.B - 1;
    const uint32_t e = key_index((uint64_t(uint32_t(__builtin_amdgcn_readlane(int(kq >> 32), bb))) << 32) |
                                 uint32_t(__builtin_amdgcn_readlane(int(uint32_t(kq)), bb)));
    ev[b] = e;
    const size_t row = size_t(h) * a.K + (e < uint32_t(a.K) ? e : 0u);
    va[b] = dd < D ? *reinterpret_cast<const float2*>(a.Abar + row * D + dd) : make_float2(0.f, 0.f);
    vl[b] = a.LSEbar[row];
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b < a.B && ev[b] < uint32_t(a.K)) {
      const size_t c = (size_t(h) * a.B + b) * a.uph + j;
      if (dd < D) *reinterpret_cast<float2*>(a.cand_a + c * D + dd) = va[b];
      if (lane == 0) a.cand_l[c] = vl[b];
    }
  }
}

// The run of scoring units this wave claims, starting with the claimed item
// v (a unit); returns the first claimed item that ends the run (a tile, a
// unit of another head, or -1).  With at most 32 sequences the queries of
// the head are loaded once and two halves stay in flight: each half's loads
// are issued before the previous half is consumed, the next claimed unit's
// first half while the current unit's second half is consumed (an item that
// ends the run loads nothing there).  Larger batches score unit by unit.
template <int D>
__device__ __forceinline__ int64_t score_run(const DecodeArgs& a, PairPool& pool, int64_t v, int SU) {
  const int SV = 2 * SU;
  if (a.B > 32) {
    while (pool_unit(pool, v)) {
      score_unit<D>(a, pool.su_lo + v, SV);
      v = claim(pool);
    }
    return v;
  }
  const int64_t u = pool.su_lo + v;
  const int h = int(u / a.uph);
  const int64_t hu = int64_t(h) * a.uph;
  u32x4 qb[2][D / 32];
  load_queries<D>(qb, a, h, 0);
  uint64_t best[2] = {0ull, 0ull};
  ScoreHalf<D> ta, tb;
  load_half<D>(ta, a, int(2 * u), SV);
  int64_t cur = u, nxt;
  for (;;) {
    load_half<D>(tb, a, int(2 * cur + 1), SV);
    __builtin_amdgcn_sched_barrier(0);
    consume_half<D>(ta, qb, a, int(64 * (cur - hu)), best);
    nxt = claim(pool);
    const int64_t un = pool.su_lo + nxt;
    const bool same = pool_unit(pool, nxt) && un / a.uph == h;
    load_half<D>(ta, a, same ? int(2 * un) : SV, SV);
    __builtin_amdgcn_sched_barrier(0);
    consume_half<D>(tb, qb, a, int(64 * (cur - hu)) + 32, best);
    store_keys<D>(a, h, int(cur - hu), 0, best);
    if (!same) break;
    cur = un;
  }
  return nxt;
}

// ---------------------------------------------------------------------------
// attention tiles: 32 tokens of one (sequence, kv head)
// ---------------------------------------------------------------------------
// Per tile and wave, everything but the softmax runs on the matrix cores:
//   S^T = K q^T   (16x16x32 bf16; A = 16 token rows of K, B = the G query
//                  rows), so lane (r16, grp) holds the scores of head r16 for
//                  the 8 tokens 4*grp + i and 16 + 4*grp + i, i < 4;
//   O += P V      (16x16x32 bf16; A = those 8 probabilities of head r16 as
//                  they lie, the k index running over the 8 tokens; B = V^T,
//                  the same 8 tokens of one head dimension, read from the
//                  row-major V tile in LDS by transposing reads).  P is split
//                  into bf16 high and low parts (two products), so it enters
//                  with about 16 significant bits while V stays exact.
// The online softmax keeps a lazy reference per head: it only moves when the
// tile maximum exceeds it by more than kLazy (base 2), so most tiles rescale
// nothing and P stays below 2^kLazy.
constexpr float kLazy = 8.0f;

template <int D, int G>
struct Tile {
  static constexpr int KS = D / 32;     // MFMA k-steps over the head dim
  static constexpr int DT = D / 16;     // 16-dim slabs of the value product
  static constexpr int LPT = D / 8;     // lanes per token row of a V load
  static constexpr int TPI = 64 / LPT;  // token rows per wave-wide V load
  static constexpr int NR = 32 / TPI;   // V rows per lane per tile
  static constexpr int kVPitch = D * 2 + 32;  // LDS bytes per V row (padded)
  static constexpr int kVBytes = 32 * kVPitch;
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

// The tile start moves the base of the tile's buffer resources (scalar
// arithmetic) and shortens their range to what is left of the segment, so the
// per-lane offsets stay loop-invariant and the loads need no vector address
// arithmetic: no temporary register can then alias a load still in flight,
// which would make the compiler drain the prefetch.  Rows past the segment end
// read as zeros; a start at or past the end loads nothing.
template <int D, int G>
__device__ __forceinline__ void load_tile(Tile<D, G>& t, const char* kseg, const char* vseg,
                                          uint32_t seg_bytes, const TileOffsets<D, G>& o,
                                          uint32_t start) {
  using T = Tile<D, G>;
  // signed difference and a maximum (scalar instructions); an unsigned
  // saturating subtract would only exist as a vector instruction, which
  // would move the resource into vector registers.  Both values stay
  // below 2^31 (the fast path bounds the segment span).
  const int rem = int(seg_bytes) - int(start);
  const uint32_t left = uint32_t(rem > 0 ? rem : 0);
  const uint32_t at = rem > 0 ? start : 0u;
  const auto rk = make_rsrc(kseg + at, left);
  const auto rv = make_rsrc(vseg + at, left);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int s = 0; s < T::KS; ++s) t.k[jj][s] = buf16_nt(rk, o.k[jj] + 64 * s, 0);
#pragma unroll
  for (int r = 0; r < T::NR; ++r) t.v[r] = buf16_nt(rv, o.v[r], 0);
}

template <int D, int G>
struct Running {
  float m, l;                  // lane (r16, *): reference and partial sum of head r16
  f32x4 o[Tile<D, G>::DT];     // lane (r16, grp): heads 4*grp + i, dim 16*dt + r16
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // nearest even
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <int D, int G>
__device__ __forceinline__ void consume_tile(const Tile<D, G>& t, Running<D, G>& st,
                                             const bf16x8 (&qb)[D / 32], float scale2,
                                             int nvalid, char* vlds) {
  using T = Tile<D, G>;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  // V rows to LDS (row-major, padded); the transposing reads below follow in
  // the same wave, whose LDS operations complete in order
  {
    const int tsub = lane / T::LPT, dd0 = 8 * (lane % T::LPT);
#pragma unroll
    for (int r = 0; r < T::NR; ++r)
      *reinterpret_cast<u32x4*>(vlds + (tsub + T::TPI * r) * T::kVPitch + dd0 * 2) = t.v[r];
  }
  f32x4 sc[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    sc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
      sc[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.k[jj][s]), qb[s], sc[jj], 0, 0, 0);
  }
  // sc[jj][i]: head r16, token 16*jj + 4*grp + i
  float mt = -INFINITY;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = 16 * jj + 4 * grp + i < nvalid;
      sc[jj][i] = ok ? sc[jj][i] * scale2 : -INFINITY;
      mt = fmaxf(mt, sc[jj][i]);
    }
  mt = group4_max(mt);  // finite: every tile holds a valid token
  const bool up = r16 < G && mt > st.m + kLazy;  // always true on the first tile
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    const float mn = up ? mt : st.m;
    const float alpha = up ? __builtin_amdgcn_exp2f(st.m - mn) : 1.0f;
    st.m = mn;
    st.l *= alpha;
    // alpha of head 4*grp + i, broadcast from lane 4*grp + i
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a0 = readlane_f(alpha, i);
      const float a1 = G > 4 ? readlane_f(alpha, 4 + i) : a0;
      al[i] = grp == 0 ? a0 : a1;
    }
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[dt][i] *= al[i];
  }
  u32x4 phi, plo;
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float p[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jj = (2 * e + h) >> 2, i = (2 * e + h) & 3;
      p[h] = __builtin_amdgcn_exp2f(sc[jj][i] - st.m);  // masked tokens: 0
      psum += p[h];
    }
    phi[e] = pack_bf16(p[0], p[1]);
    plo[e] = pack_bf16(p[0] - bf16_lo(phi[e]), p[1] - bf16_hi(phi[e]));
  }
  st.l += psum;
  wave_lds_sync();
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) {
    const bf16x8 vt = as_bf16x8(lds_read_colT(vlds, T::kVPitch, dt, 4 * grp, 16 + 4 * grp, r16));
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(phi), vt, st.o[dt], 0, 0, 0);
    st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(plo), vt, st.o[dt], 0, 0, 0);
  }
  wave_lds_sync();
}

// Segment (sequence b, kv head g) holding global tile x, from the tile
// prefix in LDS; x0 is the segment's first global tile, nt its tile count.
// n and st0 are the sequence's local length and first token slot, from the
// copies in LDS that the block took while scanning the lengths (a global load
// there would put a memory round trip in front of the segment's first tile).
struct SegLoc {
  int b, g, nt;
  int64_t x0;
  int n, st0;
};
// The sequences as the workgroup sees them, in LDS: tile prefix [B + 1],
// local lengths and first slots [B].
struct SeqTab {
  const int32_t* tp;
  const int32_t* len;
  const int32_t* st;
};
__device__ __forceinline__ SegLoc locate(const DecodeArgs& a, const SeqTab& S, int64_t x) {
  const int32_t* tp = S.tp;
  if (a.B < 64) {
    // One round of LDS reads: lane l holds sequence l's tile prefix, length
    // and first slot, and the sequence of tile x is the last one whose first
    // tile is at most x (the tile prefix does not decrease, so those lanes
    // form a prefix of the wave).  A binary search would take log2(B)
    // dependent LDS round trips, and this runs at every wave's first tile,
    // at each segment change and at the end of every pool.
    const int lane = threadIdx.x & 63;
    const int32_t tpl = tp[lane < a.B ? lane : a.B];
    const int ls = lane < a.B ? lane : a.B - 1;
    const int32_t lenl = S.len[ls], stl = S.st[ls];
    const uint64_t below = __builtin_amdgcn_ballot_w64(lane < a.B && int64_t(tpl) * a.Hkv <= x);
    const int blo = __builtin_popcountll(below) - 1;
    const int tb0 = __builtin_amdgcn_readlane(tpl, blo);
    const int nt = __builtin_amdgcn_readlane(tpl, blo + 1) - tb0;
    const int g = int((x - int64_t(tb0) * a.Hkv) / nt);
    return {blo, g, nt, int64_t(tb0) * a.Hkv + int64_t(g) * nt, __builtin_amdgcn_readlane(lenl, blo),
            __builtin_amdgcn_readlane(stl, blo)};
  }
  // LDS reads land in vector registers; readfirstlane marks the (wave-
  // uniform) values as scalars so the buffer resources built from them stay
  // in SGPRs (otherwise every buffer load becomes a waterfall loop).
  int blo = 0, bhi = a.B;  // tp[blo]*Hkv <= x < tp[bhi]*Hkv
  while (bhi - blo > 1) {
    const int mid = (blo + bhi) >> 1;
    if (int64_t(__builtin_amdgcn_readfirstlane(tp[mid])) * a.Hkv <= x) blo = mid; else bhi = mid;
  }
  const int tb0 = __builtin_amdgcn_readfirstlane(tp[blo]);
  const int nt = __builtin_amdgcn_readfirstlane(tp[blo + 1]) - tb0;
  const int g = int((x - int64_t(tb0) * a.Hkv) / nt);
  return {blo, g, nt, int64_t(tb0) * a.Hkv + int64_t(g) * nt,
          __builtin_amdgcn_readfirstlane(S.len[blo]), __builtin_amdgcn_readfirstlane(S.st[blo])};
}

// Attends the tiles of segment L that this wave claims, starting with the
// already claimed tile x (pool item v), and writes their partial state to
// `slot`.  Two register tiles are in flight: each claim's loads are issued
// before the current tile is consumed.  They are never skipped -- a claim
// outside the segment (or none) loads from past the segment end, which reads
// nothing -- so the compiler waits for exactly one tile's loads.  Returns
// the first claimed item outside the segment, or -1 once the pool is empty.
template <int D, int G>
__device__ __forceinline__ int64_t attn_run(const DecodeArgs& a, const SegLoc& L, int64_t x,
                                            PairPool& pool, int64_t slot, char* vlds) {
  int64_t nv;  // pool item of the next claim
  using T = Tile<D, G>;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int b = L.b, g = L.g;
  const int n = L.n;
  const int64_t st0 = L.st0;
  const int64_t ts = a.kv_tok_stride;
  const uint32_t seg_bytes = uint32_t(n) * uint32_t(ts) * 2u;
  const char* kseg = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.Kl) + g * a.kv_head_stride + st0 * ts));
  const char* vseg = uniform_ptr(reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.Vl) + g * a.kv_head_stride + st0 * ts));
  const TileOffsets<D, G> off(ts);
  const uint32_t tile_bytes = 32u * uint32_t(ts) * 2u;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  bf16x8 qb[T::KS];  // B operand of the score product: query rows r16 < G
#pragma unroll
  for (int s = 0; s < T::KS; ++s)
    qb[s] = as_bf16x8(r16 < G ? ld16(qp + (size_t(b) * a.Hq + g * G + r16) * D + 32 * s + 8 * grp) : zero);

  Running<D, G> st;
  st.m = r16 < G ? -INFINITY : 0.0f;  // lanes past the group hold finite filler
  st.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t x1 = L.x0 + L.nt;
  Tile<D, G> ta, tb;
  int64_t cur = x, nxt;
  load_tile<D, G>(ta, kseg, vseg, seg_bytes, off, uint32_t(cur - L.x0) * tile_bytes);
  // The scheduling barriers keep each prefetch issued before the
  // consumption of the tile already in flight; otherwise the compiler
  // hoists that tile's matrix instructions above the prefetch and has to
  // drain every load first.
  for (;;) {
    nv = claim(pool);
    nxt = pool_tile(pool, nv);
    bool in = nxt >= L.x0 && nxt < x1;
    load_tile<D, G>(tb, kseg, vseg, seg_bytes, off, in ? uint32_t(nxt - L.x0) * tile_bytes : seg_bytes);
    __builtin_amdgcn_sched_barrier(0);
    consume_tile<D, G>(ta, st, qb, a.scale2, min(32, n - 32 * int(cur - L.x0)), vlds);
    if (!in) break;
    cur = nxt;
    nv = claim(pool);
    nxt = pool_tile(pool, nv);
    in = nxt >= L.x0 && nxt < x1;
    load_tile<D, G>(ta, kseg, vseg, seg_bytes, off, in ? uint32_t(nxt - L.x0) * tile_bytes : seg_bytes);
    __builtin_amdgcn_sched_barrier(0);
    consume_tile<D, G>(tb, st, qb, a.scale2, min(32, n - 32 * int(cur - L.x0)), vlds);
    if (!in) break;
    cur = nxt;
  }

  // head totals: the denominator of head r16 summed over the lane groups
  const float lt = group4_sum(st.l);
  float* pa = a.part_a + size_t(slot) * G * D;
  float inv[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float mh = readlane_f(st.m, hh), lh = readlane_f(lt, hh);
    inv[hh] = 1.0f / lh;
    if (lane == 0) a.part_lse[size_t(slot) * G + hh] = (mh + __log2f(lh)) * ASM_LN2;
  }
  // lane (r16, grp) holds heads 4*grp + i, dims 16*dt + r16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * grp + i;
    const float iv = G > 4 ? (grp == 0 ? inv[i & (G - 1)] : inv[(4 + i) & (G - 1)]) : inv[i & (G - 1)];
    if (hh < G) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) pa[hh * D + 16 * dt + r16] = st.o[dt][i] * iv;
    }
  }
  return nv;
}

// Everything this wave claims from its pool (rank r): runs of scoring units
// and one attention piece per segment it attends; then an empty piece (lse =
// -inf, the row left as it is) for every other segment of the pool's tiles,
// so that each wave of the pair owns one slot per segment.  A wave's claims
// run contiguously from its end of the pool, so the segments it attends
// form one range.
template <int D, int G>
__device__ __forceinline__ void run_pool(const DecodeArgs& a, const SeqTab& S, PairPool& pool,
                                         int64_t r, bool disjoint, int SU, char* vlds) {
  int64_t s_lo = -1, s_hi = -2;  // segments attended
  int64_t v = claim(pool);
  while (v >= 0) {
    if (pool_unit(pool, v)) {
      v = score_run<D>(a, pool, v, SU);
      continue;
    }
    const int64_t x = pool_tile(pool, v);
    const SegLoc L = locate(a, S, x);
    const int64_t seg = int64_t(L.b) * a.Hkv + L.g;
    s_lo = s_lo < 0 ? seg : min(s_lo, seg);
    s_hi = max(s_hi, seg);
    v = attn_run<D, G>(a, L, x, pool, piece_slot(disjoint, r, seg, pool.m), vlds);
  }
  if (pool.n > pool.nsu) {
    const SegLoc F = locate(a, S, pool.t_lo), E = locate(a, S, pool.t_lo + (pool.n - pool.nsu) - 1);
    const int64_t f = int64_t(F.b) * a.Hkv + F.g, e = int64_t(E.b) * a.Hkv + E.g;
    const int lane = threadIdx.x & 63;
    for (int64_t seg = f; seg <= e; ++seg)
      if ((seg < s_lo || seg > s_hi) && lane < G)
        a.part_lse[size_t(piece_slot(disjoint, r, seg, pool.m)) * G + lane] = -INFINITY;
  }
}

// The work of wave gw in the direct layout (a wave for every potential work
// unit): scoring unit gw - (W - SU) for the last SU waves; otherwise tiles
// tpw*p .. tpw*p + tpw - 1 of segment s for gw = s * mp + p, whose partial
// state goes to slot gw (an empty one past the sequence's end).  The wave
// reads its sequence's length and first slot itself, so no wave scans the
// lengths.  `ctr` is the wave's counter in LDS.
template <int D, int G>
__device__ __forceinline__ void direct_wave(const DecodeArgs& a, int64_t gw, int32_t* ctr,
                                            char* vlds) {
  const int lane = threadIdx.x & 63;
  const int64_t W = a.n_waves;
  const int64_t SU = int64_t(a.Hq) * a.score_uph;
  const int64_t su = gw - (W - SU);
  if (su >= 0) {
    if (a.gather)
      score_unit_gather<D>(a, su, int(2 * SU));
    else
      score_unit<D>(a, su, int(2 * SU));
    return;
  }
  if (gw >= int64_t(a.B) * a.Hkv * a.mp) return;
  const int seg = int(gw / a.mp);
  const int t = int(gw - int64_t(seg) * a.mp) * a.tpw;  // first tile of this wave
  const int b = seg / a.Hkv, g = seg - b * a.Hkv;
  const int n = a.kv_len[b], st = a.kv_start[b];
  const bool valid = n >= 0 && n <= a.max_kv_len && st >= 0 && int64_t(st) + n <= a.kv_capacity;
  const int nt = valid ? (n + 31) >> 5 : 0;
  if (t >= nt) {
    if (lane < G) a.part_lse[size_t(gw) * G + lane] = -INFINITY;
    return;
  }
  // a pool of this wave's tiles (tile x = seg*mt + t ..), its first already
  // taken; the run claims the others (past the sequence's end it stops)
  const int64_t x = int64_t(seg) * a.mt + t;
  if (lane == 0) *ctr = 1;
  PairPool pool{ctr, a.tpw, 0, 0, x, 0, 1};
  const SegLoc L{b, g, nt, int64_t(seg) * a.mt, n, st};
  attn_run<D, G>(a, L, x, pool, gw, vlds);
}

}  // namespace

// Inclusive prefix sum over the 64 lanes of a wave: row shifts by 1, 2, 4
// and 8 lanes scan each row of 16 (lanes shifted in from outside the row read
// zero), then each row's total is broadcast to the rows after it.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// ---------------------------------------------------------------------------
// One workgroup (block index blk) of the main grid: NW waves.  Eight (two per
// SIMD) in general; fewer when every work unit has a wave of its own (the
// direct layout), so that the grid covers more compute units (a workgroup's
// LDS admits one eight-wave workgroup per compute unit).
template <int D, int G, int NW>
__device__ __forceinline__ void main_block(const DecodeArgs& a, int blk) {
  __shared__ int32_t tp[kFastMaxBatch + 1];
  __shared__ int32_t sq_len[kFastMaxBatch], sq_st[kFastMaxBatch];
  __shared__ int32_t wsum[NW];
  __shared__ __attribute__((aligned(16))) char vls[NW * Tile<D, G>::kVBytes];  // V tile per wave
  __shared__ int32_t ctr[NW];  // pool counters: one per pair, or one per wave (disjoint)
  // the wave index is uniform across the wave; telling the compiler keeps the
  // work-share arithmetic and the buffer resources in scalar registers
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int64_t gw = int64_t(blk) * NW + w;
  // The planner takes workgroups of fewer than eight waves exactly for the
  // direct layout (a.direct), so the workgroup size selects it at compile
  // time and the 8-wave kernel holds none of its code.
  if constexpr (NW < kMainWaves) {
    direct_wave<D, G>(a, gw, &ctr[w], vls + w * Tile<D, G>::kVBytes);
    return;
  }
  const int64_t W = a.n_waves;
  const int64_t SU = int64_t(a.Hq) * a.score_uph;
  if (threadIdx.x < NW) ctr[threadIdx.x] = 0;

  // tiles per kv head of every sequence, exclusive prefix over sequences
  if (a.B < 64) {
    // one wave scans the lengths with DPP (no LDS round trips) and the
    // workgroup meets at a single barrier
    if (w == 0) {
      int v = 0;
      if (lane < a.B) {
        const int n = a.kv_len[lane], st = a.kv_start[lane];
        sq_len[lane] = n;
        sq_st[lane] = st;
        const bool valid = n >= 0 && n <= a.max_kv_len && st >= 0 && int64_t(st) + n <= a.kv_capacity;
        v = valid ? (n + 31) >> 5 : 0;
      }
      const int x = wave_incl_scan(v);
      if (lane < a.B) tp[lane] = x - v;
      if (lane == 63) tp[a.B] = x;  // lanes past the last sequence add nothing
    }
    __syncthreads();
  } else {
    int carry = 0;
    for (int base = 0; base < a.B; base += (NW * 64)) {
      const int b = base + threadIdx.x;
      int v = 0;
      if (b < a.B) {
        const int n = a.kv_len[b], st = a.kv_start[b];
        sq_len[b] = n;
        sq_st[b] = st;
        const bool valid = n >= 0 && n <= a.max_kv_len && st >= 0 && int64_t(st) + n <= a.kv_capacity;
        v = valid ? (n + 31) >> 5 : 0;
      }
      const int x = wave_incl_scan(v);
      if (lane == 63) wsum[w] = x;
      __syncthreads();
      int before = carry;
      for (int ww = 0; ww < w; ++ww) before += wsum[ww];
      if (b < a.B) tp[b] = before + x - v;
      for (int ww = 0; ww < NW; ++ww) carry += wsum[ww];
      __syncthreads();
    }
    if (threadIdx.x == 0) tp[a.B] = carry;
    __syncthreads();
  }
  if (blk == 0)
    for (int b = threadIdx.x; b <= a.B; b += (NW * 64)) a.tile_prefix[b] = tp[b];
  const int64_t U = int64_t(__builtin_amdgcn_readfirstlane(tp[a.B])) * a.Hkv;

  // Role of this wave (plan_roles).  Attention pools go to the first Wa
  // attending ranks only, so that every pool holds at least one tile and the
  // pieces of a segment sit at consecutive ranks.
  const Roles ro = plan_roles(a, W, U);
  char* vl = vls + w * Tile<D, G>::kVBytes;
  // the pool of this wave (rank: the pair, or the wave when disjoint)
  PairPool pool{&ctr[w], 0, 0, 0, 0, 0, 0};
  int64_t rank = 0;
  if (ro.disjoint) {
    // one unit per wave, in a pool of its own
    const int64_t su = gw - (W - SU);
    if (su >= 0) {
      pool.n = pool.nsu = 1;
      pool.su_lo = su;
    } else if (gw < U) {
      rank = gw;
      pool.n = 1;
      pool.t_lo = gw;
    }
  } else {
    const int64_t P = W / 2;
    const int pw = w % (NW / 2);
    rank = int64_t(blk) * (NW / 2) + pw;
    pool.ctr = &ctr[pw];
    pool.m = w / (NW / 2);
    int64_t nt;
    if (ro.scarce) {
      const int64_t lo = share_lo(rank, ro.tot, P), hi = share_lo(rank + 1, ro.tot, P);
      pool.t_lo = min(lo, U);
      nt = min(hi, U) - pool.t_lo;
      pool.su_lo = max(lo, U) - U;
      pool.nsu = max(hi, U) - max(lo, U);
    } else {
      pool.su_lo = share_lo(rank, SU, P);
      pool.nsu = share_lo(rank + 1, SU, P) - pool.su_lo;
      nt = rank < ro.Wa ? share_lo(rank + 1, U, ro.Wa) - share_lo(rank, U, ro.Wa) : 0;
      pool.t_lo = rank < ro.Wa ? share_lo(rank, U, ro.Wa) : 0;
    }
    pool.n = pool.nsu + nt;
  }
  run_pool<D, G>(a, SeqTab{tp, sq_len, sq_st}, pool, rank, ro.disjoint, int(SU), vl);
}

template <int D, int G, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
decode_fast_main(DecodeArgs a) {
  main_block<D, G, NW>(a, int(blockIdx.x));
}

// The two-level lookup fused into the main grid: the first lookup_blocks
// workgroups run the lookup (one per sequence, head and probe rank) and the
// rest run the attention pools (scoring off).  The two roles share no
// data inside the kernel -- the lookup writes the unit keys that the combine
// reduces -- so at small batch they run side by side instead of one launch
// after the other.
template <int D, int G, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
decode_fast_main_hier(DecodeArgs a, HierArgs h, int lookup_blocks) {
  if (int(blockIdx.x) < lookup_blocks)
    hier_lookup_block<D, NW * 64>(h, int(blockIdx.x));
  else
    main_block<D, G, NW>(a, int(blockIdx.x) - lookup_blocks);
}

// The first 64 piece rows of a segment, in groups of 16 rows as far as the
// segment has pieces (rows past the last piece read as zeros through the
// buffer bounds).
template <int G>
__device__ __forceinline__ void load_piece_rows(u32x2 (&r0)[64], __amdgpu_buffer_rsrc_t rp,
                                                int64_t np, int D, int dd) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (np > 16 * j) {
#pragma unroll
      for (int i = 16 * j; i < 16 * j + 16; ++i)
        r0[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                              rp, int((i * G * D + dd) * 4), 0, 0));
    }
  }
}

// The online-softmax merge of item (b, h): the memory state (lm, am) with
// the np pieces of its segment (slots p0 .. p0 + np - 1, the first 64 rows
// already loaded in r0, their normalisers lc0 on lanes 0..63), written to
// out and out_lse.
template <int G>
__device__ __forceinline__ void merge_item(const DecodeArgs& a, int item, int hh, int D, int dd,
                                           float lm, float2 am, float lc0, const u32x2 (&r0)[64],
                                           int64_t p0, int64_t np, __amdgpu_buffer_rsrc_t rp) {
  const int lane = threadIdx.x & 63;
  float* o = a.out + size_t(item) * D;
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
  // an empty piece (weight 0) may hold stale values: skip it
  const auto acc = [&](float wi, const u32x2& r) {
    v0 = wi > 0.0f ? fmaf(wi, __uint_as_float(r[0]), v0) : v0;
    v1 = wi > 0.0f ? fmaf(wi, __uint_as_float(r[1]), v1) : v1;
  };
  const float wc0 = lc0 == -INFINITY ? 0.0f : expf(lc0 - M);
  float zsum = wc0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (np > 16 * j) {
#pragma unroll
      for (int i = 16 * j; i < 16 * j + 16; ++i) acc(readlane_f(wc0, i), r0[i]);
    }
  }
  for (int64_t c64 = 64; c64 < np; c64 += 64) {
    const float lc = c64 + lane < np ? a.part_lse[(p0 + c64 + lane) * G + hh] : -INFINITY;
    const float wc = lc == -INFINITY ? 0.0f : expf(lc - M);
    zsum += wc;
    const int64_t cend = min<int64_t>(np, c64 + 64);
    for (int64_t c = c64; c < cend; c += 16) {
      u32x2 r[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        r[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             rp, int(((c + i) * G * D + dd) * 4), 0, 0));
#pragma unroll
      for (int i = 0; i < 16; ++i) acc(readlane_f(wc, int(c - c64) + i), r[i]);
    }
  }
  const float Z = wm + wave_sum(zsum);
  const float inv = 1.0f / Z;
  if (dd < D) *reinterpret_cast<float2*>(o + dd) = make_float2(v0 * inv, v1 * inv);
  if (lane == 0 && a.out_lse) a.out_lse[item] = M + logf(Z);
}

// One wave per (b, h): index from the unit keys, gather of the memory
// state, merge with the partial states of segment (b, h / G).  The loads are
// arranged in two dependent rounds: (1) sequence bounds, tile prefix, keys;
// (2) the gathered memory state, the piece normalisers and up to 64 piece
// rows (rows past the last piece read as zeros through the buffer bounds);
// later pieces, if any, follow 16 rows at a time.
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
  if (!a.no_memory)
    for (int u = lane; u < a.uph; u += 64) best = umax64(best, kk[u]);
  const int nt = tpb1 - tpb;
  int64_t p0 = 0, np = 0;  // pieces of segment (b, g)
  if (nt > 0) {
    const int64_t total = int64_t(tpB) * a.Hkv;
    const Roles ro = plan_roles(a, a.n_waves, total);
    const int64_t first = int64_t(tpb) * a.Hkv + int64_t(g) * nt;
    const int64_t seg = int64_t(b) * a.Hkv + g;
    const int64_t r0 = wave_of(first, ro.tot, ro.Wt), r1 = wave_of(first + nt - 1, ro.tot, ro.Wt);
    p0 = piece_slot(ro.disjoint, r0, seg, 0);
    np = (ro.disjoint ? 1 : 2) * (r1 - r0 + 1);
  }
  best = wave_max_u64(best);
  const uint32_t k = a.no_memory ? 0u : __builtin_amdgcn_readfirstlane(key_index(best));
  if (lane == 0 && a.out_idx) a.out_idx[item] = int32_t(k);
  float* o = a.out + size_t(item) * D;
  const int dd = 2 * lane;
  // the pieces must lie in the workspace's partial-state rows (they do
  // whenever the main grid of this step ran on this workspace; a tile
  // prefix it did not write must not send the loads elsewhere)
  const int64_t pieces = int64_t(a.n_waves) + 2 * int64_t(a.B) * a.Hkv;
  const bool placed = nt >= 0 && p0 >= 0 && np >= 0 && p0 + np <= pieces;
  if (!valid || !placed || k >= uint32_t(a.K)) {
    if (dd < D) *reinterpret_cast<float2*>(o + dd) = make_float2(NAN, NAN);
    if (lane == 0 && a.out_lse) a.out_lse[item] = NAN;
    return;
  }
  // round 2
  const float lm = a.no_memory ? -INFINITY : a.LSEbar[size_t(h) * a.K + k];
  const float2 am = (dd < D && !a.no_memory)
                        ? *reinterpret_cast<const float2*>(a.Abar + (size_t(h) * a.K + k) * D + dd)
                        : make_float2(0.f, 0.f);
  const float* pa0 = a.part_a + (p0 * G + hh) * D;
  const auto rp = make_rsrc(pa0, np > 0 ? uint32_t(((np - 1) * G + 1) * D * 4) : 0u);
  // the first 64 piece normalisers and piece rows load with the memory state;
  // a segment split over many waves (a long context at small batch) thus
  // merges its first 64 pieces after one round
  const float lc0 = lane < np ? a.part_lse[(p0 + lane) * G + hh] : -INFINITY;
  u32x2 r0[64];
  load_piece_rows<G>(r0, rp, np, D, dd);
  merge_item<G>(a, item, hh, D, dd, lm, am, lc0, r0, p0, np, rp);
}

// The merge in the direct layout: segment (b, g)'s pieces are slots
// (b*Hkv + g)*mp .. +mp (those past the sequence's end empty), known without
// the tile prefix, so they load in the first round with the keys; with
// gathering, so do the units' candidate states, and the winner's state is the
// candidate of the unit that holds the winning entry.  One dependent round of
// loads in all (two without gathering: the memory state).  One wave per
// workgroup: a step this small has few items, and one wave per compute unit
// keeps each unit's share of the item loads small.
template <int G>
__global__ void __launch_bounds__(64) decode_fast_combine_direct(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x;
  if (item >= a.B * a.Hq) return;
  const int b = item / a.Hq, h = item % a.Hq;
  const int g = h / G, hh = h % G;
  const int D = a.d;
  const int dd = 2 * lane;
  const bool valid = seq_valid(a, b);
  const uint64_t* kk = a.keys + (size_t(h) * a.B + b) * a.uph;
  uint64_t best = 0;
  if (!a.no_memory)
    for (int u = lane; u < a.uph; u += 64) best = umax64(best, kk[u]);
  const int64_t p0 = (int64_t(b) * a.Hkv + g) * a.mp, np = a.mp;
  const float* pa0 = a.part_a + (p0 * G + hh) * D;
  const auto rp = make_rsrc(pa0, np > 0 ? uint32_t(((np - 1) * G + 1) * D * 4) : 0u);
  const float lc0 = lane < np ? a.part_lse[(p0 + lane) * G + hh] : -INFINITY;
  u32x2 r0[64];
  load_piece_rows<G>(r0, rp, np, D, dd);
  // candidates: unit j's best entry state for this (h, b), j < uph <= 16
  u32x2 cr[16];
  float cl = -INFINITY;
  if (a.gather) {
    const size_t c0 = (size_t(h) * a.B + b) * a.uph;
    const auto rc = make_rsrc(a.cand_a + c0 * D, uint32_t(a.uph) * D * 4);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      cr[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, int((j * D + dd) * 4), 0, 0));
    cl = lane < a.uph ? a.cand_l[c0 + lane] : -INFINITY;
  }
  best = wave_max_u64(best);
  const uint32_t k = a.no_memory ? 0u : __builtin_amdgcn_readfirstlane(key_index(best));
  if (lane == 0 && a.out_idx) a.out_idx[item] = int32_t(k);
  if (!valid || k >= uint32_t(a.K)) {
    float* o = a.out + size_t(item) * D;
    if (dd < D) *reinterpret_cast<float2*>(o + dd) = make_float2(NAN, NAN);
    if (lane == 0 && a.out_lse) a.out_lse[item] = NAN;
    return;
  }
  float lm = -INFINITY;
  float2 am = make_float2(0.f, 0.f);
  if (!a.no_memory) {
    if (a.gather) {
      const int js = int(k >> 6);  // the unit holding entry k
      u32x2 sel = cr[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) sel = j == js ? cr[j] : sel;
      lm = readlane_f(cl, js);
      if (dd < D) am = make_float2(__uint_as_float(sel[0]), __uint_as_float(sel[1]));
    } else {
      lm = a.LSEbar[size_t(h) * a.K + k];
      if (dd < D) am = *reinterpret_cast<const float2*>(a.Abar + (size_t(h) * a.K + k) * D + dd);
    }
  }
  merge_item<G>(a, item, hh, D, dd, lm, am, lc0, r0, p0, np, rp);
}

// ---------------------------------------------------------------------------
bool decode_fast_path(int dtype, int d, int G, int K, int64_t kv_tok_stride, int max_kv_len) {
  // buffer offsets are 32-bit: one sequence's KV rows and one head's
  // centroid rows (plus a 64-row unit past the end) must span < 2 GiB
  const bool fits = int64_t(max_kv_len + 32) * kv_tok_stride * 2 < (int64_t(1) << 31) &&
                    (int64_t(K) + 64) * d * 2 < (int64_t(1) << 31);
  return dtype == 0 && (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8) && fits;
}

template <int D, int G>
static void launch_fast_hier(const DecodeArgs& a, const HierArgs& h, hipStream_t s) {
  const int lookup_blocks = a.B * a.Hq * h.p;
  if (a.wg_waves == kSmallWaves)
    hipLaunchKernelGGL((decode_fast_main_hier<D, G, kHierSmallWaves>),
                       dim3(unsigned(lookup_blocks + a.n_waves / kHierSmallWaves)), dim3(kHierSmallWaves * 64),
                       0, s, a, h, lookup_blocks);
  else
    hipLaunchKernelGGL((decode_fast_main_hier<D, G, kMainWaves>),
                       dim3(unsigned(lookup_blocks + a.n_waves / kMainWaves)), dim3(kMainThreads), 0,
                       s, a, h, lookup_blocks);
  if (a.direct)
    hipLaunchKernelGGL((decode_fast_combine_direct<G>), dim3(a.B * a.Hq), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((decode_fast_combine<G>), dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
}

// phase bit 1: the main grid; bit 2: the merge
template <int D, int G>
static void launch_fast(const DecodeArgs& a, hipStream_t s, int phase = 3) {
  if (phase & 1) {
    if (a.wg_waves == kSmallWaves)
      hipLaunchKernelGGL((decode_fast_main<D, G, kSmallWaves>), dim3(a.n_waves / kSmallWaves),
                         dim3(kSmallWaves * 64), 0, s, a);
    else
      hipLaunchKernelGGL((decode_fast_main<D, G, kMainWaves>), dim3(a.n_waves / kMainWaves),
                         dim3(kMainThreads), 0, s, a);
  }
  if (phase & 2) {
    if (a.direct)
      hipLaunchKernelGGL((decode_fast_combine_direct<G>), dim3(a.B * a.Hq), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((decode_fast_combine<G>), dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, s, a);
  }
}

template <int D, int G>
static int occupancy_waves() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_fast_main<D, G, kMainWaves>, kMainThreads, 0) !=
          hipSuccess || blocks < 1)
    blocks = 1;
  return kMainWaves * blocks;
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

static hipError_t launch_fast_phase(const DecodeArgs& a, hipStream_t s, int phase) {
  const int G = a.Hq / a.Hkv;
  if (a.d == 128) {
    switch (G) {
      case 1: launch_fast<128, 1>(a, s, phase); break;
      case 2: launch_fast<128, 2>(a, s, phase); break;
      case 4: launch_fast<128, 4>(a, s, phase); break;
      default: launch_fast<128, 8>(a, s, phase); break;
    }
  } else {
    switch (G) {
      case 1: launch_fast<64, 1>(a, s, phase); break;
      case 2: launch_fast<64, 2>(a, s, phase); break;
      case 4: launch_fast<64, 4>(a, s, phase); break;
      default: launch_fast<64, 8>(a, s, phase); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s) { return launch_fast_phase(a, s, 3); }
hipError_t launch_decode_fast_main(const DecodeArgs& a, hipStream_t s) { return launch_fast_phase(a, s, 1); }
hipError_t launch_decode_fast_merge(const DecodeArgs& a, hipStream_t s) { return launch_fast_phase(a, s, 2); }

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

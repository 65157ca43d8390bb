// Prefix attention states on MFMA (bf16 inputs, d in {64, 128}, GQA group
// G in {1, 2, 4, 8}).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Calibración Offline -- Recolección (per
// calibration query, the attention state over the prefix) and Eficiencia
// (the prefix is cut into chunks whose states are merged with the
// online-softmax identity).
//
// A workgroup holds eight waves (two per SIMD, so one wave's softmax overlaps
// the other's matrix work) that share one kv head's K/V tiles: wave w
// computes the states of 32 queries of one query head.  Per 64-key tile:
//   S^T = K Q^T      (16x16x32 bf16 MFMA; A = K rows from LDS, B = the
//                     wave's queries in registers), so every lane's scores
//                     belong to one query column and the online softmax
//                     needs no register transposes;
//   O^T += V^T P^T   (16x16x32 f16 MFMA; A = V^T, gathered from the
//                     row-major fp16 V tile in LDS by transposing reads
//                     (ds_read_b64_tr_b16), B = the probabilities, already
//                     in the B-operand layout);
//   l += 1^T P^T     (the same MFMA with an all-ones A operand), so the
//                     softmax denominator is the sum of exactly the fp16
//                     probabilities that enter O, summed on the matrix
//                     cores instead of the vector ALUs.
// The softmax runs once per 64-key tile (one maximum, reduced across the
// wave's four 16-lane groups with the gfx950 lane-swap instructions).  The
// probability-value products run in fp16: P < 2^8 (lazy maximum, below) and
// fp16 keeps 3 more mantissa bits than bf16; V is converted to fp16 once per
// call into the workspace, so its values must stay below 65504.  At each
// chunk boundary the chunk state (O/l, m + log l) is written (if requested)
// and merged into the running state, which lives in the output (A, LSE)
// between chunks: every wave reads back only rows it wrote itself.
#include "common.hpp"
#include "kernels.hpp"
#include "states_generic.hpp"

namespace asmk {

namespace {

constexpr int kKeys = 64;        // keys per LDS tile
constexpr int kQ = 32;           // queries per wave (two MFMA column tiles)
constexpr int kWaves = 8;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;

template <int D>
struct StatesSmem {
  // padded K row (bf16): 32 bytes past a multiple of 256 keeps the 16-byte
  // operand reads of 16 rows free of LDS bank conflicts (measured on gfx950;
  // +16 loses about half of the LDS cycles to conflicts)
  static constexpr int kKRow = D * 2 + 32;
  static constexpr int kVRow = D * 2 + 32;           // padded V row (fp16)
  static constexpr int kKBytes = kKeys * kKRow;
  static constexpr int kVBytes = kKeys * kVRow;
  static constexpr int kBuf = kKBytes + kVBytes;
  static constexpr int kBytes = 2 * kBuf;
  static constexpr int kKChunks = kKeys * D / 8 / kThreads;  // 16-byte K pieces per thread
  static constexpr int kVChunks = kKeys * D / 8 / kThreads;
};

template <int D>
struct Staged {
  u32x4 k[StatesSmem<D>::kKChunks];
  u32x4 v[StatesSmem<D>::kVChunks];
};

// global -> registers for the tile starting at key k0 (keys past L read zeros)
template <int D>
__device__ __forceinline__ void stage_load(Staged<D>& r, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, int k0) {
  constexpr int kPieces = D / 8;
#pragma unroll
  for (int i = 0; i < StatesSmem<D>::kKChunks; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int key = c / kPieces, piece = c % kPieces;
    r.k[i] = buf16(rk, ((k0 + key) * D + piece * 8) * 2, 0);
  }
#pragma unroll
  for (int i = 0; i < StatesSmem<D>::kVChunks; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int key = c / kPieces, piece = c % kPieces;
    r.v[i] = buf16(rv, ((k0 + key) * D + piece * 8) * 2, 0);
  }
}

// registers -> LDS: K row-major [key][d] (bf16), V row-major [key][d] (fp16)
template <int D>
__device__ __forceinline__ void stage_store(char* buf, const Staged<D>& r) {
  using S = StatesSmem<D>;
  constexpr int kPieces = D / 8;
#pragma unroll
  for (int i = 0; i < S::kKChunks; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int key = c / kPieces, piece = c % kPieces;
    *reinterpret_cast<u32x4*>(buf + key * S::kKRow + piece * 16) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < S::kVChunks; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int key = c / kPieces, piece = c % kPieces;
    *reinterpret_cast<u32x4*>(buf + S::kKBytes + key * S::kVRow + piece * 16) = r.v[i];
  }
}

// V^T operand of the value MFMA for dims 16*dt .. +15 and the 8 keys
// {kb .. kb+3} and {kb2 .. kb2+3} (per lane group) of the tile in LDS.
template <int D>
__device__ __forceinline__ f16x8 load_vt(const char* vbase, int dt, int kb, int kb2, int r16) {
  return __builtin_bit_cast(f16x8, lds_read_colT(vbase, StatesSmem<D>::kVRow, dt, kb, kb2, r16));
}

// bf16 -> fp16 (round to nearest even), eight values per thread.  A finite
// value of magnitude 65520 or more has no fp16 form (it would become
// infinity); then the flag is raised and the states kernel takes its exact
// bf16 path instead.
__global__ void v_to_f16_kernel(const u32x4* src, u32x4* dst, int64_t n8, int* overflow) {
  bool ovf = false;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n8;
       i += int64_t(gridDim.x) * blockDim.x) {
    const u32x4 v = src[i];
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(v[e]), x1 = bf16_hi(v[e]);
      const _Float16 lo = (_Float16)x0;
      const _Float16 hi = (_Float16)x1;
      ovf |= (__builtin_isinf(float(lo)) && !__builtin_isinf(x0)) ||
             (__builtin_isinf(float(hi)) && !__builtin_isinf(x1));
      o[e] = uint32_t(__builtin_bit_cast(uint16_t, lo)) | (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    dst[i] = o;
  }
  if (__builtin_amdgcn_ballot_w64(ovf) != 0 && (threadIdx.x & 63) == 0) atomicOr(overflow, 1);
}

__global__ void clear_flag(int* flag) { *flag = 0; }

}  // namespace

// Online softmax of one 64-key tile for query column tile qt: scores
// st[ks][kk][qt][i] belong to key 32*ks + 16*kk + 4*grp + i.  The reference
// maximum m is lazy: it only moves when the tile's maximum exceeds it by more
// than kLazy (base-2 units), so most tiles rescale nothing; the
// probabilities then stay below 2^kLazy, far inside fp16.  Exponents are
// exp2(s * scale2 - m) with one rounding (scale2 > 0).  Returns whether m
// moved (then O must be scaled by alpha[qt]).
constexpr float kLazy = 8.0f;

template <bool kFull>
__device__ __forceinline__ bool softmax_tile(const f32x4 (&st)[2][2][2], int qt, int grp,
                                             int nvalid, float scale2, float (&m)[2],
                                             float (&alpha)[2], f16x8 (&pb)[2][2]) {
  float mt = -INFINITY;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = kFull || 32 * ks + 16 * kk + 4 * grp + i < nvalid;
        mt = fmaxf(mt, ok ? st[ks][kk][qt][i] : -INFINITY);
      }
  mt = group4_max(mt);
  const float mts = mt * scale2;
  const bool up = mts > m[qt] + kLazy;  // always true for the first tile
  const float mn = up ? mts : m[qt];
  alpha[qt] = up ? __builtin_amdgcn_exp2f(m[qt] - mn) : 1.0f;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = kFull || 32 * ks + 16 * kk + 4 * grp + i < nvalid;
        const float p = ok ? __builtin_amdgcn_exp2f(fmaf(st[ks][kk][qt][i], scale2, -mn)) : 0.0f;
        pb[ks][qt][4 * kk + i] = (_Float16)p;
      }
  m[qt] = mn;
  return up;
}

// GW query heads per workgroup share the K/V tiles (GW = min(G, 4)); the
// workgroup covers 32 * 8 / GW queries of each of its heads.
template <int D, int GW>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
states_mfma_kernel(StatesArgs a, int row_blocks, int hsubs) {
  using S = StatesSmem<D>;
  constexpr int KS = D / 32;   // k-steps of the score MFMA
  constexpr int DT = D / 16;   // dim tiles of the value MFMA
  __shared__ __attribute__((aligned(16))) char smem[S::kBytes];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, grp = lane >> 4;
  const int G = a.Hq / a.Hkv;

  const int rb = blockIdx.x % row_blocks;
  const int hs = (blockIdx.x / row_blocks) % hsubs;
  const int g = blockIdx.x / (row_blocks * hsubs);
  const int h = g * G + hs * GW + (w % GW);
  const int q0 = rb * (kQ * kWaves / GW) + kQ * (w / GW);  // first query of this wave

  // A value with no fp16 form: this wave's queries take the exact bf16 path
  // (the flag is the same for the whole grid, so no barrier is skipped by
  // only part of a workgroup).
  if (__builtin_amdgcn_readfirstlane(*a.v_overflow) != 0) {
    for (int q = q0; q < q0 + kQ && q < a.N; ++q) states_one_query<uint16_t>(a, h, q);
    return;
  }

  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.Kp) + size_t(g) * a.L * D, uint32_t(a.L) * D * 2);
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.V16) + size_t(g) * a.L * D, uint32_t(a.L) * D * 2);
  const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + size_t(h) * a.N * D, uint32_t(a.N) * D * 2);

  // B operand of the score MFMA: query columns q0 + 16*qt + r16 (past N: zeros)
  bf16x8 qb[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qb[qt][s] = as_bf16x8(buf16(rq, ((q0 + 16 * qt + r16) * D + 32 * s + 8 * grp) * 2, 0));

  const bool acc_in = a.accumulate != 0;

  float O[DT][2][4];
  f32x4 lacc[2];  // per query column: sum of the (fp16) probabilities, in every row
  float m[2];
  const f16x8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  Staged<D> stg;
  int buf_i = 0;
  bool have_tile = false;
  const int nc = a.nc;
  for (int c = 0; c < nc; ++c) {
    const int c_lo = c * a.chunk, c_hi = min(a.L, (c + 1) * a.chunk);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      m[qt] = -INFINITY;
      lacc[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[dt][qt][i] = 0.0f;
    }
    if (!have_tile) {  // first tile of the whole prefix
      stage_load<D>(stg, rk, rv, c_lo);
      stage_store<D>(smem, stg);
      have_tile = true;
    }
    for (int k0 = c_lo; k0 < c_hi; k0 += kKeys) {
      __syncthreads();  // tile k0 is in buffer buf_i; the other buffer is free
      char* cur = smem + buf_i * S::kBuf;
      // the next tile: next keys of this chunk, else the first of the next
      // chunk; after the last tile the loads start at L and read zeros.  The
      // loads and the LDS store are never skipped, so the compiler's wait
      // for them stays at the store.
      const int nk = k0 + kKeys < c_hi ? k0 + kKeys : c_hi;
      stage_load<D>(stg, rk, rv, nk);
      const int nvalid = min(kKeys, c_hi - k0);
      // scores of the whole tile: st[ks][kk][qt] for keys 32*ks + 16*kk + 4*grp + i
      // and query column r16 of tile qt
      f32x4 st[2][2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 ka[KS];
#pragma unroll
          for (int s = 0; s < KS; ++s)
            ka[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                cur + (32 * ks + 16 * kk + r16) * S::kKRow + (32 * s + 8 * grp) * 2));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            st[ks][kk][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
              st[ks][kk][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[qt][s], st[ks][kk][qt], 0, 0, 0);
          }
        }
      f16x8 pb[2][2];
      float alpha[2];
      const bool up0 = nvalid >= kKeys
                           ? softmax_tile<true>(st, 0, grp, nvalid, a.scale2, m, alpha, pb)
                           : softmax_tile<false>(st, 0, grp, nvalid, a.scale2, m, alpha, pb);
      const bool up1 = nvalid >= kKeys
                           ? softmax_tile<true>(st, 1, grp, nvalid, a.scale2, m, alpha, pb)
                           : softmax_tile<false>(st, 1, grp, nvalid, a.scale2, m, alpha, pb);
      if (__any(up0 || up1)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[dt][qt][i] *= alpha[qt];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i) lacc[qt][i] *= alpha[qt];
      }
      // O^T += V^T P^T over the tile's 64 keys; the k index of lane group grp
      // in half ks is keys 32*ks + {4grp..4grp+3} then 32*ks + 16 + {4grp..4grp+3},
      // matching pb[ks]
      const char* vbase = cur + S::kKBytes;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f16x8 va = load_vt<D>(vbase, dt, 32 * ks + 4 * grp, 32 * ks + 16 + 4 * grp, r16);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            f32x4 o = {O[dt][qt][0], O[dt][qt][1], O[dt][qt][2], O[dt][qt][3]};
            o = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[ks][qt], o, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) O[dt][qt][i] = o[i];
          }
        }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          lacc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[ks][qt], lacc[qt], 0, 0, 0);
      stage_store<D>(smem + (buf_i ^ 1) * S::kBuf, stg);
      buf_i ^= 1;
    }
    // chunk state and running merge (per query column r16 of each qt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float lt = lacc[qt][0];
      const bool empty = m[qt] == -INFINITY;
      const float inv = empty ? 0.0f : 1.0f / lt;
      const float lse_c = empty ? -INFINITY : (m[qt] + __log2f(lt)) * ASM_LN2;
      const int q = q0 + 16 * qt + r16;
      if (a.A_chunks && q < a.N) {
        const size_t row = (size_t(c) * a.Hq + h) * a.N + q;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = O[dt][qt][i] * inv;
          *reinterpret_cast<f32x4*>(a.A_chunks + row * D + 16 * dt + 4 * grp) = v;
        }
        if (grp == 0) a.LSE_chunks[row] = lse_c;
      }
      // merge into the running state kept in (A, LSE); chunk 0 of a fresh
      // build has no running state
      if (q < a.N) {
        const size_t row = size_t(h) * a.N + q;
        const bool fresh = c == 0 && !acc_in;
        const float lr = fresh ? -INFINITY : a.LSE[row];
        const float M = fmaxf(lr, lse_c);
        const float w1 = lr == -INFINITY ? 0.0f : expf(lr - M);
        const float w2 = empty ? 0.0f : expf(lse_c - M);
        const float z = w1 + w2;
        const float iz = M == -INFINITY ? 0.0f : 1.0f / z;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          float* ap = a.A + row * D + 16 * dt + 4 * grp;
          const f32x4 r = fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(ap);
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (w1 * r[i] + w2 * O[dt][qt][i] * inv) * iz;
          *reinterpret_cast<f32x4*>(ap) = v;
        }
        if (grp == 0) a.LSE[row] = M == -INFINITY ? -INFINITY : M + logf(z);
      }
    }
  }
}

bool states_fast_path(int dtype, int d, int G) {
  return dtype == 0 && (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

size_t states_v16_bytes(int Hkv, int L, int d) { return (size_t(Hkv) * L * d * 2 + 255) / 256 * 256; }

size_t states_ws_bytes(int dtype, int Hq, int Hkv, int N, int L, int d) {
  if (!states_fast_path(dtype, d, Hq / Hkv) || L == 0 || N == 0) return 0;
  if (int64_t(L + kKeys) * d * 2 >= (int64_t(1) << 31) || int64_t(N + kQ * kWaves) * d * 2 >= (int64_t(1) << 31))
    return 0;
  return states_v16_bytes(Hkv, L, d) + 256;  // fp16 V, then the overflow flag
}

template <int D, int GW>
static void launch_states(const StatesArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int rows = kQ * kWaves / GW;
  const int row_blocks = (a.N + rows - 1) / rows;
  const int hsubs = G / GW;
  const dim3 grid(unsigned(row_blocks * hsubs * a.Hkv));
  hipLaunchKernelGGL((states_mfma_kernel<D, GW>), grid, dim3(kThreads), 0, s, a, row_blocks, hsubs);
}

hipError_t launch_build_states(const StatesArgs& a, int dtype, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (states_ws_bytes(dtype, a.Hq, a.Hkv, a.N, a.L, a.d) == 0 || a.V16 == nullptr ||
      a.v_overflow == nullptr || !(a.scale2 > 0.0f))
    return launch_states_generic(a, dtype, s);
  const int64_t n8 = int64_t(a.Hkv) * a.L * a.d / 8;
  const int64_t vb = (n8 + 255) / 256;
  hipLaunchKernelGGL(clear_flag, dim3(1), dim3(1), 0, s, a.v_overflow);
  hipLaunchKernelGGL(v_to_f16_kernel, dim3(unsigned(vb < 8192 ? vb : 8192)), dim3(256), 0, s,
                     static_cast<const u32x4*>(a.Vp), static_cast<u32x4*>(a.V16), n8, a.v_overflow);
  if (a.d == 128) {
    if (G == 1) launch_states<128, 1>(a, s);
    else if (G == 2) launch_states<128, 2>(a, s);
    else launch_states<128, 4>(a, s);
  } else {
    if (G == 1) launch_states<64, 1>(a, s);
    else if (G == 2) launch_states<64, 2>(a, s);
    else launch_states<64, 4>(a, s);
  }
  return hipGetLastError();
}

}  // namespace asmk

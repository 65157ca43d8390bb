// Prefix attention states on MFMA (bf16 inputs, d in {64, 128}, GQA group
// G in {1, 2, 4, 8}).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Calibración Offline -- Recolección (per
// calibration query, the attention state over the prefix) and Eficiencia
// (the prefix is cut into chunks whose states are merged with the
// online-softmax identity).
//
// A workgroup holds four waves that share one kv head's K/V tiles: wave w
// computes the states of 32 queries of one query head.  Per 64-key tile:
//   S^T = K Q^T      (16x16x32 bf16 MFMA; A = K rows from LDS, B = the
//                     wave's queries in registers), so every lane's scores
//                     belong to one query column and the online softmax
//                     needs no register transposes;
//   O^T += V^T P^T   (16x16x32 f16 MFMA; A = V^T read from an LDS copy of the
//                     tile transposed to [dim][key] in fp16, B = the
//                     probabilities, already in the B-operand layout).
// The probability-value products run in fp16: P <= 1 and fp16 keeps 3 more
// mantissa bits than bf16; V values must stay below 65504.  At each chunk
// boundary the chunk state (O/l, m + log l) is written (if requested) and
// merged into the running state in registers.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

namespace {

constexpr int kKeys = 64;        // keys per LDS tile
constexpr int kQ = 32;           // queries per wave (two MFMA column tiles)

template <int D>
struct StatesSmem {
  static constexpr int kKRow = D * 2 + 16;           // padded K row (bf16)
  static constexpr int kVRow = kKeys * 2 + 8;        // padded V^T row (fp16)
  static constexpr int kKBytes = kKeys * kKRow;
  static constexpr int kVBytes = D * kVRow;
  static constexpr int kBuf = kKBytes + kVBytes;
  static constexpr int kBytes = 2 * kBuf;
  static constexpr int kKChunks = kKeys * D / 8 / 256;  // 16-byte K pieces per thread
  static constexpr int kVChunks = kKeys * D / 8 / 256;
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
    const int c = threadIdx.x + 256 * i;
    const int key = c / kPieces, piece = c % kPieces;
    r.k[i] = buf16(rk, ((k0 + key) * D + piece * 8) * 2, 0);
  }
#pragma unroll
  for (int i = 0; i < StatesSmem<D>::kVChunks; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int key = c % kKeys, dd0 = 8 * (c / kKeys);
    r.v[i] = buf16(rv, ((k0 + key) * D + dd0) * 2, 0);
  }
}

// registers -> LDS: K row-major [key][d] (bf16); V transposed [d][key] (fp16)
template <int D>
__device__ __forceinline__ void stage_store(char* buf, const Staged<D>& r) {
  using S = StatesSmem<D>;
  constexpr int kPieces = D / 8;
#pragma unroll
  for (int i = 0; i < S::kKChunks; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int key = c / kPieces, piece = c % kPieces;
    *reinterpret_cast<u32x4*>(buf + key * S::kKRow + piece * 16) = r.k[i];
  }
  _Float16* vt = reinterpret_cast<_Float16*>(buf + S::kKBytes);
#pragma unroll
  for (int i = 0; i < S::kVChunks; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int key = c % kKeys, dd0 = 8 * (c / kKeys);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(dd0 + 2 * e) * (S::kVRow / 2) + key] = (_Float16)bf16_lo(r.v[i][e]);
      vt[(dd0 + 2 * e + 1) * (S::kVRow / 2) + key] = (_Float16)bf16_hi(r.v[i][e]);
    }
  }
}

}  // namespace

// GW query heads per workgroup share the K/V tiles (GW = min(G, 4)); the
// workgroup covers 32 * 4 / GW queries of each of its heads.
template <int D, int GW>
__global__ void __launch_bounds__(256) states_mfma_kernel(StatesArgs a, int row_blocks, int hsubs) {
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
  const int q0 = rb * (kQ * 4 / GW) + kQ * (w / GW);  // first query of this wave

  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.Kp) + size_t(g) * a.L * D, uint32_t(a.L) * D * 2);
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.Vp) + size_t(g) * a.L * D, uint32_t(a.L) * D * 2);
  const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + size_t(h) * a.N * D, uint32_t(a.N) * D * 2);

  // B operand of the score MFMA: query columns q0 + 16*qt + r16 (past N: zeros)
  bf16x8 qb[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qb[qt][s] = as_bf16x8(buf16(rq, ((q0 + 16 * qt + r16) * D + 32 * s + 8 * grp) * 2, 0));

  // running (merged) state, O^T layout: dim 16*dt + 4*grp + i, query 16*qt + r16
  float R[DT][2][4];
  float lseR[2];
  const bool acc_in = a.accumulate != 0;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q0 + 16 * qt + r16;
    const bool qv = q < a.N;
    lseR[qt] = (acc_in && qv) ? a.LSE[size_t(h) * a.N + q] : -INFINITY;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        R[dt][qt][i] = (acc_in && qv) ? a.A[(size_t(h) * a.N + q) * D + 16 * dt + 4 * grp + i] : 0.0f;
  }

  float O[DT][2][4];
  float m[2], l[2];
  Staged<D> stg;
  int buf_i = 0;
  bool have_tile = false;
  const int nc = a.nc;
  for (int c = 0; c < nc; ++c) {
    const int c_lo = c * a.chunk, c_hi = min(a.L, (c + 1) * a.chunk);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      m[qt] = -INFINITY;
      l[qt] = 0.0f;
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
      // the next tile: next keys of this chunk, else the first of the next chunk
      const int nk = k0 + kKeys < c_hi ? k0 + kKeys : (c + 1 < nc ? c_hi : -1);
      if (nk >= 0) stage_load<D>(stg, rk, rv, nk);
      const int nvalid = min(kKeys, c_hi - k0);
#pragma unroll
      for (int ks = 0; ks < kKeys / 32; ++ks) {
        // scores of keys 32*ks + 16*kk + 4*grp + i (kk = 0, 1) for query column r16
        f32x4 st[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 ka[KS];
#pragma unroll
          for (int s = 0; s < KS; ++s)
            ka[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                cur + (32 * ks + 16 * kk + r16) * S::kKRow + (32 * s + 8 * grp) * 2));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            st[kk][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
              st[kk][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qb[qt][s], st[kk][qt], 0, 0, 0);
          }
        }
        f16x8 pb[2];
        bool rescale = false;
        float alpha[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          float sv[2][4];
          float mt = -INFINITY;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = 32 * ks + 16 * kk + 4 * grp + i;
              sv[kk][i] = key < nvalid ? st[kk][qt][i] * a.scale2 : -INFINITY;
              mt = fmaxf(mt, sv[kk][i]);
            }
          mt = fmaxf(mt, shfl_xor_f(mt, 16));
          mt = fmaxf(mt, shfl_xor_f(mt, 32));
          const float mn = fmaxf(m[qt], mt);
          // a block of only masked keys (mn = -inf) leaves the state alone
          alpha[qt] = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m[qt] - mn);
          rescale |= alpha[qt] != 1.0f;
          float lp = 0.0f;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[kk][i] - mn);
              lp += p;
              pb[qt][4 * kk + i] = (_Float16)p;
            }
          l[qt] = l[qt] * alpha[qt] + lp;
          m[qt] = mn;
        }
        if (__any(rescale)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
              for (int i = 0; i < 4; ++i) O[dt][qt][i] *= alpha[qt];
        }
        // O^T += V^T P^T over these 32 keys; the k index of lane group grp is
        // keys {4grp..4grp+3} then {16+4grp..16+4grp+3}, matching pb
        const _Float16* vt = reinterpret_cast<const _Float16*>(cur + S::kKBytes);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const _Float16* row = vt + (16 * dt + r16) * (S::kVRow / 2) + 32 * ks + 4 * grp;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16);
          const u32x4 vv = {lo[0], lo[1], hi[0], hi[1]};
          const f16x8 va = __builtin_bit_cast(f16x8, vv);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            f32x4 o = {O[dt][qt][0], O[dt][qt][1], O[dt][qt][2], O[dt][qt][3]};
            o = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[qt], o, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) O[dt][qt][i] = o[i];
          }
        }
      }
      if (nk >= 0) stage_store<D>(smem + (buf_i ^ 1) * S::kBuf, stg);
      buf_i ^= 1;
    }
    // chunk state and running merge (per query column r16 of each qt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float lt = l[qt];
      lt += shfl_xor_f(lt, 16);
      lt += shfl_xor_f(lt, 32);
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
      const float M = fmaxf(lseR[qt], lse_c);
      if (M != -INFINITY) {
        const float w1 = lseR[qt] == -INFINITY ? 0.0f : expf(lseR[qt] - M);
        const float w2 = empty ? 0.0f : expf(lse_c - M);
        const float z = w1 + w2;
        const float iz = 1.0f / z;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) R[dt][qt][i] = (w1 * R[dt][qt][i] + w2 * O[dt][qt][i] * inv) * iz;
        lseR[qt] = M + logf(z);
      }
    }
  }
  // merged state
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = q0 + 16 * qt + r16;
    if (q >= a.N) continue;
    const size_t row = size_t(h) * a.N + q;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = lseR[qt] == -INFINITY ? 0.0f : R[dt][qt][i];
      *reinterpret_cast<f32x4*>(a.A + row * D + 16 * dt + 4 * grp) = v;
    }
    if (grp == 0) a.LSE[row] = lseR[qt];
  }
}

bool states_fast_path(int dtype, int d, int G) {
  return dtype == 0 && (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

template <int D, int GW>
static void launch_states(const StatesArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int rows = kQ * 4 / GW;
  const int row_blocks = (a.N + rows - 1) / rows;
  const int hsubs = G / GW;
  const dim3 grid(unsigned(row_blocks * hsubs * a.Hkv));
  hipLaunchKernelGGL((states_mfma_kernel<D, GW>), grid, dim3(256), 0, s, a, row_blocks, hsubs);
}

hipError_t launch_build_states(const StatesArgs& a, int dtype, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const bool fits = int64_t(a.L + kKeys) * a.d * 2 < (int64_t(1) << 31) &&
                    int64_t(a.N + kQ * 4) * a.d * 2 < (int64_t(1) << 31);
  if (!states_fast_path(dtype, a.d, G) || !fits || a.L == 0 || a.N == 0)
    return launch_states_generic(a, dtype, s);
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

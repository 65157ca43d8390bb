// k-means assignment on MFMA (bf16, d in {64, 128}).
//
// Source: "Context Memorization for Efficient Long Context Generation"
// (technical summary), Fase de Calibración Offline -- Agrupamiento (the
// collected queries are clustered); the metric is the retrieval cosine of
// Fase de Inferencia Online -- Recuperación.
//
// idx[h,i] = argmax_k X[h,i].C[h,k] * cinv[h,k] (lowest k on exact ties) is a
// GEMM X C^T with a row argmax fused into its epilogue, so the N x K score
// matrix never leaves registers.  One workgroup owns 256 query rows (64 per
// wave, held in registers as MFMA A operands) and streams the head's whole
// centroid table through LDS in double-buffered tiles of 64 centroids.  The
// small tiles (35 KB of LDS) and a 168-register budget let three waves share
// each SIMD, so one wave's argmax epilogue overlaps another's MFMAs.  Each
// lane keeps, for each of its 16 rows, the best score seen in its column
// slot; a DPP reduction over the 16 lanes of a row finishes the argmax.
// Workgroups are mapped XCD-aware: each XCD walks a contiguous range of
// (head, row block) pairs, so one head's table stays hot in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

namespace {

constexpr int kRowsPerWave = 64;              // 4 MFMA row tiles of 16
constexpr int kRowsPerWG = 4 * kRowsPerWave;  // 256
constexpr int kTileCols = 64;                 // centroids per LDS tile
constexpr int kXcds = 8;

template <int D>
struct AssignSmem {
  // padded centroid row: a pitch of 32 bytes past a multiple of 256 spreads
  // the 16-byte operand reads of 16 rows over all LDS banks (measured on
  // gfx950: no bank conflicts, against half the LDS cycles lost at +16)
  static constexpr int kRowBytes = D * 2 + 32;
  static constexpr int kTileBytes = kTileCols * kRowBytes;
  static constexpr int kBufBytes = kTileBytes + kTileCols * 4;  // rows + inverse norms
  static constexpr int kBytes = 2 * kBufBytes;
};

template <int D>
__device__ __forceinline__ void stage_tile(char* buf, __amdgpu_buffer_rsrc_t rc,
                                           __amdgpu_buffer_rsrc_t ri, int k0, int K,
                                           u32x4 (&reg)[kTileCols * D * 2 / 16 / 256], float& ci) {
  // global -> registers: chunk c of the tile is row c / (D/8), 16-byte piece c % (D/8)
  constexpr int kChunksPerRow = D / 8;
  constexpr int kPer = kTileCols * kChunksPerRow / 256;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / kChunksPerRow, piece = c % kChunksPerRow;
    reg[i] = buf16(rc, ((k0 + row) * D + piece * 8) * 2, 0);
  }
  // columns past K get a NaN inverse norm: their scores are NaN and never win
  ci = threadIdx.x < kTileCols ? (k0 + int(threadIdx.x) < K ? buf_f32(ri, (k0 + threadIdx.x) * 4, 0) : __builtin_nanf("")) : 0.0f;
  (void)buf;
}

template <int D>
__device__ __forceinline__ void commit_tile(char* buf, const u32x4 (&reg)[kTileCols * D * 2 / 16 / 256],
                                            float ci) {
  constexpr int kChunksPerRow = D / 8;
  constexpr int kPer = kTileCols * kChunksPerRow / 256;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / kChunksPerRow, piece = c % kChunksPerRow;
    *reinterpret_cast<u32x4*>(buf + row * AssignSmem<D>::kRowBytes + piece * 16) = reg[i];
  }
  if (threadIdx.x < kTileCols)
    reinterpret_cast<float*>(buf + AssignSmem<D>::kTileBytes)[threadIdx.x] = ci;
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
assign_mfma_kernel(AssignArgs a, int row_blocks, int per_xcd) {
  constexpr int KS = D / 32;
  constexpr int kPer = kTileCols * (D / 8) / 256;
  __shared__ __attribute__((aligned(16))) char smem[AssignSmem<D>::kBytes];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, grp = lane >> 4;

  // XCD-aware work mapping: blockIdx % 8 is the XCD, and each XCD walks a
  // contiguous range of (head, row block) pairs.
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int gidx = xcd * per_xcd + local;
  if (gidx >= a.H * row_blocks) return;
  const int h = gidx / row_blocks, rb = gidx % row_blocks;
  const int row0 = rb * kRowsPerWG + w * kRowsPerWave;

  const auto rx = make_rsrc(static_cast<const uint16_t*>(a.X) + size_t(h) * a.N * D, uint32_t(a.N) * D * 2);
  const auto rc = make_rsrc(static_cast<const uint16_t*>(a.C) + size_t(h) * a.K * D, uint32_t(a.K) * D * 2);
  const auto ri = make_rsrc(a.cinv + size_t(h) * a.K, uint32_t(a.K) * 4);

  // A operands: rows row0 + 16*rt + r16, d chunk 32*s + 8*grp (rows past N are zeros)
  u32x4 xa[4][KS];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int s = 0; s < KS; ++s) xa[rt][s] = buf16(rx, ((row0 + 16 * rt + r16) * D + 32 * s + 8 * grp) * 2, 0);

  float best[4][4];
  int bidx[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      best[rt][i] = -INFINITY;
      bidx[rt][i] = 0;
    }

  const int ntiles = (a.K + kTileCols - 1) / kTileCols;
  u32x4 reg[kPer];
  float ci;
  stage_tile<D>(smem, rc, ri, 0, a.K, reg, ci);
  commit_tile<D>(smem, reg, ci);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // tile kt is in buffer kt % 2; buffer (kt+1) % 2 is free
    char* cur = smem + (kt & 1) * AssignSmem<D>::kBufBytes;
    char* nxt = smem + ((kt + 1) & 1) * AssignSmem<D>::kBufBytes;
    if (kt + 1 < ntiles) stage_tile<D>(nxt, rc, ri, (kt + 1) * kTileCols, a.K, reg, ci);
    const float* cil = reinterpret_cast<const float*>(cur + AssignSmem<D>::kTileBytes);
#pragma unroll 1  // unrolling raises the register count past three waves per SIMD
    for (int ct = 0; ct < kTileCols / 16; ++ct) {
      // B operand: centroid column ct*16 + r16, d chunk 32*s + 8*grp
      bf16x8 cb[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        cb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(cur + (ct * 16 + r16) * AssignSmem<D>::kRowBytes +
                                                          (32 * s + 8 * grp) * 2));
      const int col = kt * kTileCols + ct * 16 + r16;
      const float cv = cil[ct * 16 + r16];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[rt][s]), cb[s], acc, 0, 0, 0);
        // acc[i]: row 16*rt + 4*grp + i against column `col`; columns are
        // visited in increasing order, so a strict > keeps the lowest index
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sc = acc[i] * cv;
          const bool take = sc > best[rt][i];
          best[rt][i] = take ? sc : best[rt][i];
          bidx[rt][i] = take ? col : bidx[rt][i];
        }
      }
    }
    if (kt + 1 < ntiles) commit_tile<D>(nxt, reg, ci);
  }

  // finish each row across the 16 lanes of its DPP row: highest score, then
  // lowest index among exact ties
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m = row16_max(best[rt][i]);
      int cand = best[rt][i] == m ? bidx[rt][i] : 0x7FFFFFFF;
      cand = min(cand, __builtin_amdgcn_update_dpp(0x7FFFFFFF, cand, kDppQuadXor1, 0xF, 0xF, false));
      cand = min(cand, __builtin_amdgcn_update_dpp(0x7FFFFFFF, cand, kDppQuadXor2, 0xF, 0xF, false));
      cand = min(cand, __builtin_amdgcn_update_dpp(0x7FFFFFFF, cand, kDppRowRor4, 0xF, 0xF, false));
      cand = min(cand, __builtin_amdgcn_update_dpp(0x7FFFFFFF, cand, kDppRowRor8, 0xF, 0xF, false));
      const int row = row0 + 16 * rt + 4 * grp + i;
      if (r16 == 0 && row < a.N) {
        const size_t o = size_t(h) * a.N + row;
        a.idx[o] = cand == 0x7FFFFFFF ? 0 : cand;
        if (a.best) a.best[o] = m;
      }
    }
}

bool assign_fast_path(int dtype, int d) { return dtype == 0 && (d == 64 || d == 128); }

hipError_t launch_assign(const AssignArgs& a, int dtype, hipStream_t s) {
  if (!assign_fast_path(dtype, a.d) || int64_t(a.K) * a.d * 2 >= (int64_t(1) << 31) ||
      int64_t(a.N) * a.d * 2 >= (int64_t(1) << 31))
    return launch_assign_generic(a, dtype, s);
  const int row_blocks = (a.N + kRowsPerWG - 1) / kRowsPerWG;
  const int total = a.H * row_blocks;
  if (total == 0) return hipSuccess;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const dim3 grid(unsigned(per_xcd * kXcds));
  if (a.d == 128)
    hipLaunchKernelGGL(assign_mfma_kernel<128>, grid, dim3(256), 0, s, a, row_blocks, per_xcd);
  else
    hipLaunchKernelGGL(assign_mfma_kernel<64>, grid, dim3(256), 0, s, a, row_blocks, per_xcd);
  return hipGetLastError();
}

}  // namespace asmk

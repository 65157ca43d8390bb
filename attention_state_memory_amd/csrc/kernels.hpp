// Argument blocks and launchers shared between the HIP kernels and the C ABI
// layer.  Every launcher enqueues on the given stream and returns the result
// of hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace asmk {

// ---- decode step ----------------------------------------------------------
// Two workspace layouts exist.  The MFMA path (bf16, d in {64, 128},
// Hq/Hkv in {1, 2, 4, 8}) balances the step over a persistent grid of
// n_waves waves; the plain VALU path splits each sequence into fixed token
// splits.
struct DecodeArgs {
  int B, Hq, Hkv, d, K;
  float scale2;  // softmax scale * log2(e): scores are kept as base-2 logits
  const void* q;   // [B, Hq, d] the queries the local attention uses
  const void* qs;  // [B, Hq, d] the queries the lookup scores: q, or q whitened
  const void* C;
  const float* cinv;
  const float* Abar;
  const float* LSEbar;
  const void* Kl;
  const void* Vl;
  int64_t kv_head_stride, kv_tok_stride, kv_capacity;
  const int32_t* kv_start;
  const int32_t* kv_len;
  int max_kv_len;
  float* out;
  float* out_lse;
  int32_t* out_idx;
  // MFMA path (the planner's choice: n_waves > 0)
  int n_waves;           // persistent waves (multiple of kMainWaves); 0 on the VALU path
  int wg_waves;          // waves per workgroup of the main launch: kMainWaves, or
                         // kSmallWaves when every work unit has a wave of its own
  int uph;               // argmax keys per (head, sequence): ceil(K / 64) units
  int score_uph;         // units per head the main kernel scores: uph, or 0 when
                         // the keys were written beforehand (hierarchical lookup)
  int32_t* tile_prefix;  // [B + 1] 32-token tiles per kv head, prefix over sequences
  int no_memory;         // attention only: no lookup, the merge starts from the empty state
  // VALU path
  int split_tok;    // local tokens per attention item
  int S_max;        // splits per sequence = ceil(max_kv_len / split_tok)
  int score_tiles;  // ceil(K / 256)
  // both
  uint64_t* keys;   // MFMA: [Hq, B, uph]; VALU: [Hq, score_tiles, B]
  float* part_a;    // MFMA: [n_waves + 2*B*Hkv, G, d]; VALU: [B, Hq, S_max, d]
  float* part_lse;  // MFMA: [n_waves + 2*B*Hkv, G];    VALU: [B, Hq, S_max]
  // (last, so that the fields above keep their kernel-argument offsets)
  // direct layout (grids with a wave for every potential work unit): tiles
  // tpw*p .. tpw*p + tpw - 1 of segment s (sequence b, kv head g;
  // s = b*Hkv + g) are wave and partial slot s*mp + p, so neither kernel
  // needs the lengths' prefix
  int direct;
  int mt;                // ceil(max_kv_len / 32): potential tiles per segment
  int tpw;               // direct: tiles per wave (and per partial slot)
  int mp;                // direct: pieces per segment, ceil(mt / tpw)
  int gather;            // direct, at most 16 units per head and 8 sequences: each
                         // scoring unit also gathers its best entry's state
  float* cand_a;         // gather: [Hq, B, uph, d] state of each unit's best entry
  float* cand_l;         // gather: [Hq, B, uph] its lse
};

constexpr int kFastMaxBatch = 2048;  // sequences per MFMA-path launch
constexpr int kMainWaves = 8;        // waves per workgroup of the MFMA main grid (two per SIMD)
constexpr int kMainThreads = 64 * kMainWaves;
// waves per workgroup when the grid has a wave per work unit (the direct
// layout): one, so that the grid spreads over as many compute units as it
// has waves; four in the two-level kernel, whose lookup workgroups share
// the launch and need at least 128 threads
constexpr int kSmallWaves = 1;
constexpr int kHierSmallWaves = 4;
bool decode_fast_path(int dtype, int d, int G, int K, int64_t kv_tok_stride, int max_kv_len);
int decode_fast_waves_per_cu(int d, int G);  // resident waves per CU of the MFMA main kernel
hipError_t launch_decode_fast(const DecodeArgs& a, hipStream_t s);
// the two launches of launch_decode_fast, for callers that split the step:
// the main grid (scoring, lookup keys, local attention -> partial states),
// then the merge
hipError_t launch_decode_fast_main(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_fast_merge(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t s);

// ---- hierarchical lookup ------------------------------------------------------
constexpr int kHierMaxProbes = 32;
constexpr int kHierMaxSupers = 1024;
struct HierArgs {
  int B, Hq, K, S, d, p;
  const void* q;        // [B, Hq, d]
  const void* C;        // [Hq, K, d]
  const float* cinv;    // [Hq, K]
  const void* SC;       // [Hq, S, d] super-centroids
  const float* scinv;   // [Hq, S]
  const int32_t* offsets;  // [Hq, S + 1]
  const int32_t* members;  // [Hq, K]
  const void* Cg;       // [Hq, K, d] nullable: C[h, members[h, i]] at row i (grouped by super)
  const float* cginv;   // [Hq, K] nullable: cinv in the same order
  uint64_t* keys;       // [Hq, B, p] one argmax key per (head, sequence, probe)
  int32_t* probes_out;  // [B, Hq, p] nullable
};
bool hier_fast_path(int dtype, int d);
// Cg[h, i] = C[h, members[h, i]], cginv[h, i] = cinv[h, members[h, i]] (a
// zero row and 0 for a member outside [0, K))
hipError_t launch_index_group_rows(int dtype, int H, int K, int d, const void* C, const float* cinv,
                                   const int32_t* members, void* Cg, float* cginv, hipStream_t s);
// the main grid with the lookup fused in (MFMA path only), then the combine
hipError_t launch_decode_hier(const DecodeArgs& a, const HierArgs& h, hipStream_t s);

// ---- whitening at retrieval ---------------------------------------------------
struct WhitenFitArgs {
  int H, N, d, nblk, max_iters;
  double ridge;
  const void* X;       // [H, N, d] calibration queries
  double* part_mean;   // [H, nblk, d] workspace
  double* part_cov;    // [H, nblk, d, d] workspace
  double* mats;        // [H, 4, d, d] workspace (iteration matrices)
  double* mu;          // [H, d]
  double* W;           // [H, d, d]
  double* resid;       // [H] |Z Y - I|_F at exit, nullable
};
struct WhitenRowsArgs {
  int H, d;
  int64_t M;                        // rows per head
  int64_t head_stride, row_stride;  // elements, shared by Y and Yw
  const void* Y;
  void* Yw;
  const double* mu;  // [H, d]
  const double* W;   // [H, d, d]
};
int whiten_blocks(int H, int N);
size_t whiten_fit_ws_bytes(int H, int N, int d);
hipError_t launch_whiten_fit(WhitenFitArgs a, int dtype, hipStream_t s);
hipError_t launch_whiten_rows(const WhitenRowsArgs& a, int dtype, hipStream_t s);

// ---- centroid inverse norms -------------------------------------------------
hipError_t launch_inv_norms(int dtype, int H, int K, int d, const void* C, float* cinv,
                            hipStream_t s);

// ---- prefix states ------------------------------------------------------------
struct StatesArgs {
  int Hq, Hkv, N, L, d, chunk, nc;
  float scale2;
  const void* Q;
  const void* Kp;
  const void* Vp;
  float* A_chunks;
  float* LSE_chunks;
  float* A;
  float* LSE;
  int accumulate;
  void* V16;        // MFMA path: Vp converted to fp16 [Hkv, L, d] (workspace)
  int* v_overflow;  // MFMA path: set when a finite Vp value has no fp16 form (workspace)
};
bool states_fast_path(int dtype, int d, int G);
size_t states_ws_bytes(int dtype, int Hq, int Hkv, int N, int L, int d);  // 0: VALU path
size_t states_v16_bytes(int Hkv, int L, int d);  // the fp16 V part of that workspace
hipError_t launch_build_states(const StatesArgs& a, int dtype, hipStream_t s);
hipError_t launch_states_generic(const StatesArgs& a, int dtype, hipStream_t s);

// ---- k-means assignment -----------------------------------------------------
struct AssignArgs {
  int H, N, K, d;
  const void* X;
  const void* C;
  const float* cinv;
  int32_t* idx;
  float* best;
};
bool assign_fast_path(int dtype, int d);
hipError_t launch_assign(const AssignArgs& a, int dtype, hipStream_t s);
hipError_t launch_assign_generic(const AssignArgs& a, int dtype, hipStream_t s);

// ---- aggregation ------------------------------------------------------------
struct AggregateArgs {
  int H, N, K, d;
  const void* X;
  const int32_t* idx;
  const float* A;
  const float* LSE;
  void* C;
  float* cinv;
  int32_t* count;
  float* Abar;
  float* LSEbar;
  int32_t* offsets;  // [H, K+1] workspace
  int32_t* cursor;   // [H, K]   workspace
  int32_t* perm;     // [H, N]   workspace
  int32_t* part;     // [H, nchunks, K] workspace for the LDS counting sort, or NULL
};
constexpr int kAggChunk = 4096;      // queries per counting-sort workgroup
constexpr int kAggLdsMaxK = 16384;   // largest K whose counters fit in LDS
inline int agg_chunks(int N) { return (N + kAggChunk - 1) / kAggChunk; }
hipError_t launch_aggregate(const AggregateArgs& a, int dtype, hipStream_t s);

}  // namespace asmk

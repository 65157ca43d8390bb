// C ABI of the attention-state-memory library: argument validation,
// workspace layout and kernel dispatch.  Declarations and the contract of
// every entry point are in include/asm_memory.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "asm_memory.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return ASM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ASM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dtype(int dtype) {
  if (dtype != ASM_BF16 && dtype != ASM_F32) return fail(ASM_ERR_DTYPE, "unknown dtype %d", dtype);
  return ASM_OK;
}

int check_d(int dtype, int d) {
  if (d < 1 || d > 256) return fail(ASM_ERR_SHAPE, "head dim d=%d outside 1..256", d);
  if (dtype == ASM_BF16 && d % 8 != 0)
    return fail(ASM_ERR_SHAPE, "bf16 head dim d=%d is not a multiple of 8", d);
  return ASM_OK;
}

int check_bf16_ptrs(int dtype, std::initializer_list<const void*> ptrs) {
  if (dtype != ASM_BF16) return ASM_OK;
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(ASM_ERR_ALIGN, "bf16 tensor %p is not 16-byte aligned", p);
  return ASM_OK;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return ASM_OK;
  if (ws == nullptr) return fail(ASM_ERR_WORKSPACE, "workspace of %zu bytes required, ws is NULL", need);
  if (ws_bytes < need)
    return fail(ASM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0)
    return fail(ASM_ERR_ALIGN, "workspace %p is not 16-byte aligned", ws);
  return ASM_OK;
}

#define ASM_TRY(expr)          \
  do {                         \
    const int st_ = (expr);    \
    if (st_ != ASM_OK) return st_; \
  } while (0)

// ---- decode planning -------------------------------------------------------
// Direct layout (small steps): local tiles per wave and per partial state.
constexpr int kDirectTilesPerWave = 2;
struct DecodePlan {
  bool fast = false;
  int Bc = 0;  // sequences per launch
  int n_waves = 0, wg_waves = 0, uph = 0, score_uph = 0;  // MFMA path
  int direct = 0, mt = 0, tpw = 1, mp = 0, gather = 0;    // MFMA path, small steps
  size_t off_ca = 0, off_cl = 0;
  int split_tok = 0, S_max = 0, score_tiles = 0;  // VALU path
  size_t off_keys = 0, off_tp = 0, off_pa = 0, off_pl = 0, total = 0;
};

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

int decode_split_tokens(int B, int Hkv, int max_kv_len) {
  // about 2048 attention items per step
  const int64_t work = int64_t(B) * Hkv * max_kv_len;
  int64_t s = (work + 2047) / 2048;
  s = (s + 127) / 128 * 128;
  if (s < 128) s = 128;
  if (s > 4096) s = 4096;
  return int(s);
}

// keys_given > 0: that many argmax keys per (head, sequence) come from the
// two-level lookup (one per probe), so the main kernel scores nothing.
DecodePlan plan_decode(int dtype, int B, int Hq, int Hkv, int d, int K, int max_kv_len,
                       int64_t kv_tok_stride, int keys_given = 0) {
  DecodePlan p;
  const int G = Hq / Hkv;
  p.fast = asmk::decode_fast_path(dtype, d, G, K, kv_tok_stride, max_kv_len);
  const int Bc = B < asmk::kFastMaxBatch ? B : asmk::kFastMaxBatch;
  const int uph = keys_given > 0 ? keys_given : (K + 63) / 64;
  const int score_uph = keys_given > 0 ? 0 : uph;
  const int64_t units = int64_t(Hq) * score_uph + int64_t(Bc) * Hkv * ((int64_t(max_kv_len) + 31) / 32);
  // the pools count their claims and index scoring halves in 32 bits
  if (units >= (int64_t(1) << 30)) p.fast = false;
  size_t off = 0;
  if (p.fast) {
    p.Bc = Bc;
    p.uph = uph;
    p.score_uph = score_uph;
    // Persistent grid: as many waves as fit on the device at once, but no
    // more than one per work unit (16 KB each): small steps are latency-bound
    // and gain from spreading their few units over many waves.
    const int64_t cap = int64_t(device_cus()) * asmk::decode_fast_waves_per_cu(d, G);
    int64_t w = units;
    w = w < cap ? w : cap;
    if (w < 2) w = 2;
    w = (w + asmk::kMainWaves - 1) / asmk::kMainWaves * asmk::kMainWaves;
    p.n_waves = int(w);
    // The direct layout (a wave for every unit, whatever the actual lengths;
    // one-wave workgroups spread the grid over more compute units) when the
    // persistent grid is not capped, and also when scoring dominates the
    // step: local attention waves at most a quarter of the scoring units
    // (measured at batch 1-4 with K=8192 and batch 2 with K=32768: 8-17%
    // faster; at half or more the pools win, up to 1.4x at 32 sequences).
    const int64_t attn_waves = int64_t(Bc) * Hkv *
        (((int64_t(max_kv_len) + 31) / 32 + kDirectTilesPerWave - 1) / kDirectTilesPerWave);
    const bool direct = w >= units || 4 * attn_waves <= int64_t(Hq) * score_uph;
    p.wg_waves = direct ? asmk::kSmallWaves : asmk::kMainWaves;
    // With a wave for every potential unit, tile t of segment s is wave and
    // slot s * mt + t (direct layout: no scan of the lengths); with at most
    // 16 units per head and 8 sequences, the scoring units also gather their
    // best entries' states, so the merge needs one round of loads.
    p.direct = p.wg_waves == asmk::kSmallWaves ? 1 : 0;
    p.mt = int((int64_t(max_kv_len) + 31) / 32);
    p.tpw = kDirectTilesPerWave;
    p.mp = (p.mt + p.tpw - 1) / p.tpw;
    if (p.direct) {
      // the direct layout's waves: the scoring units and ceil(mt / tpw) per
      // segment (fewer workgroups to dispatch than one wave per tile)
      int64_t wd = int64_t(Hq) * score_uph + int64_t(Bc) * Hkv * p.mp;
      if (wd < 2) wd = 2;
      p.n_waves = int((wd + asmk::kMainWaves - 1) / asmk::kMainWaves * asmk::kMainWaves);
    }
    p.gather = p.direct && score_uph > 0 && score_uph <= 16 && p.Bc <= 8 ? 1 : 0;
    p.off_keys = off;
    off = asmk::align_up(off + size_t(Hq) * p.Bc * p.uph * sizeof(uint64_t), kAlign);
    p.off_tp = off;
    off = asmk::align_up(off + size_t(p.Bc + 1) * sizeof(int32_t), kAlign);
    // one partial state per (rank, segment), two per rank when ranks are wave
    // pairs; the direct layout: one per attention wave
    const size_t pieces = p.direct ? size_t(p.Bc) * Hkv * p.mp
                                   : size_t(p.n_waves) + 2 * size_t(p.Bc) * Hkv;
    p.off_pa = off;
    off = asmk::align_up(off + pieces * G * d * sizeof(float), kAlign);
    p.off_pl = off;
    off = asmk::align_up(off + pieces * G * sizeof(float), kAlign);
    if (p.gather) {
      p.off_ca = off;
      off = asmk::align_up(off + size_t(Hq) * p.Bc * p.uph * d * sizeof(float), kAlign);
      p.off_cl = off;
      off = asmk::align_up(off + size_t(Hq) * p.Bc * p.uph * sizeof(float), kAlign);
    }
  } else {
    p.Bc = B;
    p.split_tok = decode_split_tokens(B, Hkv, max_kv_len);
    p.S_max = max_kv_len > 0 ? (max_kv_len + p.split_tok - 1) / p.split_tok : 0;
    p.score_tiles = (K + 255) / 256;
    p.off_keys = off;
    off = asmk::align_up(off + size_t(Hq) * p.score_tiles * B * sizeof(uint64_t), kAlign);
    p.off_pa = off;
    off = asmk::align_up(off + size_t(B) * Hq * p.S_max * d * sizeof(float), kAlign);
    p.off_pl = off;
    off = asmk::align_up(off + size_t(B) * Hq * p.S_max * sizeof(float), kAlign);
  }
  p.total = off;
  return p;
}

int validate_decode_shape(int dtype, int B, int Hq, int Hkv, int d, int K, int max_kv_len) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (B < 1 || Hq < 1 || Hkv < 1 || K < 1 || max_kv_len < 0)
    return fail(ASM_ERR_SHAPE, "need B, Hq, Hkv, K >= 1 and max_kv_len >= 0 (B=%d Hq=%d Hkv=%d K=%d max_kv_len=%d)",
                B, Hq, Hkv, K, max_kv_len);
  if (Hq % Hkv != 0) return fail(ASM_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int64_t items = int64_t(B) * Hkv * ((int64_t(max_kv_len) + 127) / 128) + int64_t(Hq) * ((K + 255) / 256);
  if (items > (int64_t(1) << 30) || int64_t(B) * Hq > (int64_t(1) << 30))
    return fail(ASM_ERR_SHAPE, "decode problem too large for one launch");
  return ASM_OK;
}

// Host checks of a decode step's arguments (no device call).
int check_decode_args(int dtype, int B, int Hq, int Hkv, int d, int K, float scale, const void* q,
                      const void* C, const float* cinv, const float* Abar, const float* LSEbar,
                      const void* Kl, const void* Vl, int64_t kv_head_stride,
                      int64_t kv_tok_stride, int64_t kv_capacity, const int32_t* kv_start,
                      const int32_t* kv_len, int max_kv_len, const float* out,
                      bool attend_only) {
  ASM_TRY(validate_decode_shape(dtype, B, Hq, Hkv, d, K, max_kv_len));
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(ASM_ERR_SHAPE, "scale must be finite");
  if (attend_only) {
    if (!q || !kv_start || !kv_len || !out)
      return fail(ASM_ERR_NULL, "q, kv_start, kv_len and out are required");
  } else if (!q || !C || !cinv || !Abar || !LSEbar || !kv_start || !kv_len || !out) {
    return fail(ASM_ERR_NULL, "q, C, cinv, Abar, LSEbar, kv_start, kv_len and out are required");
  }
  if (max_kv_len > 0) {
    if (!Kl || !Vl) return fail(ASM_ERR_NULL, "Kl and Vl are required when max_kv_len > 0");
    if (kv_head_stride < 0 || kv_tok_stride < 1 || kv_capacity < 0)
      return fail(ASM_ERR_SHAPE, "need kv_head_stride >= 0, kv_tok_stride >= 1, kv_capacity >= 0");
    if (dtype == ASM_BF16 && (kv_head_stride % 8 != 0 || kv_tok_stride % 8 != 0))
      return fail(ASM_ERR_ALIGN, "bf16 kv strides must be multiples of 8 elements");
  }
  ASM_TRY(check_bf16_ptrs(dtype, {q, C, Kl, Vl}));
  return ASM_OK;
}

// The decode step for every lookup; `hier` (hierarchical lookup) is NULL for
// the flat search; `qs` (the queries the lookup scores) is NULL when they are
// the queries themselves.  `phase`: 3 the whole step; 1 its first launch
// (the main grid), 2 its second (the merge), for the flat MFMA path in one
// launch.
int decode_impl(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                const void* q, const void* C, const float* cinv, const float* Abar,
                const float* LSEbar, const void* Kl, const void* Vl,
                int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                float* out, float* out_lse, int32_t* out_idx,
                void* ws, size_t ws_bytes, hipStream_t stream, asmk::HierArgs* hier,
                const void* qs = nullptr, bool attend_only = false, int phase = 3) {
  ASM_TRY(check_decode_args(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                            kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len,
                            max_kv_len, out, attend_only));
  const DecodePlan p = plan_decode(dtype, B, Hq, Hkv, d, K, max_kv_len, kv_tok_stride,
                                   hier != nullptr ? hier->p : (attend_only ? 1 : 0));
  if (attend_only && !p.fast)
    return fail(ASM_ERR_SHAPE,
                "attention without memory needs bf16, d in {64, 128}, Hq/Hkv in {1, 2, 4, 8}, "
                "KV rows of under 2 GiB per sequence and under 2^30 work units per launch");
  if (hier != nullptr && !p.fast)
    return fail(ASM_ERR_SHAPE,
                "the hierarchical lookup needs bf16, d in {64, 128}, Hq/Hkv in {1, 2, 4, 8}, "
                "local KV rows of under 2 GiB per sequence and under 2^30 work units per launch");
  if (phase != 3 && (!p.fast || hier != nullptr || attend_only || B > p.Bc))
    return fail(ASM_ERR_SHAPE,
                "the decode in two launches needs bf16, d in {64, 128}, Hq/Hkv in {1, 2, 4, 8}, "
                "KV rows of under 2 GiB per sequence and at most %d sequences",
                asmk::kFastMaxBatch);
  ASM_TRY(check_ws(ws, ws_bytes, p.total));

  asmk::DecodeArgs a{};
  a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.K = K;
  a.scale2 = scale * ASM_LOG2E;
  a.C = C; a.cinv = cinv; a.Abar = Abar; a.LSEbar = LSEbar;
  a.Kl = Kl; a.Vl = Vl;
  a.kv_head_stride = kv_head_stride; a.kv_tok_stride = kv_tok_stride; a.kv_capacity = kv_capacity;
  a.max_kv_len = max_kv_len;
  a.no_memory = attend_only ? 1 : 0;
  a.n_waves = p.n_waves; a.wg_waves = p.wg_waves; a.uph = p.uph; a.score_uph = p.score_uph;
  a.direct = p.direct; a.mt = p.mt; a.tpw = p.tpw; a.mp = p.mp; a.gather = p.gather;
  a.split_tok = p.split_tok; a.S_max = p.S_max; a.score_tiles = p.score_tiles;
  char* w = static_cast<char*>(ws);
  a.keys = reinterpret_cast<uint64_t*>(w + p.off_keys);
  a.tile_prefix = reinterpret_cast<int32_t*>(w + p.off_tp);
  a.part_a = reinterpret_cast<float*>(w + p.off_pa);
  a.part_lse = reinterpret_cast<float*>(w + p.off_pl);
  a.cand_a = p.gather ? reinterpret_cast<float*>(w + p.off_ca) : nullptr;
  a.cand_l = p.gather ? reinterpret_cast<float*>(w + p.off_cl) : nullptr;
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  int32_t* probes_base = hier ? hier->probes_out : nullptr;
  // Sequences are independent: batches larger than one launch's limit run
  // as consecutive launches over batch slices sharing the workspace.
  for (int b0 = 0; b0 < B; b0 += p.Bc) {
    const int nb = B - b0 < p.Bc ? B - b0 : p.Bc;
    a.B = nb;
    a.q = static_cast<const char*>(q) + size_t(b0) * Hq * d * esz;
    a.qs = qs ? static_cast<const char*>(qs) + size_t(b0) * Hq * d * esz : a.q;
    a.kv_start = kv_start + b0;
    a.kv_len = kv_len + b0;
    a.out = out + size_t(b0) * Hq * d;
    a.out_lse = out_lse ? out_lse + size_t(b0) * Hq : nullptr;
    a.out_idx = out_idx ? out_idx + size_t(b0) * Hq : nullptr;
    if (hier != nullptr) {
      hier->B = nb;
      hier->q = a.q;
      hier->keys = a.keys;
      hier->probes_out = probes_base ? probes_base + size_t(b0) * Hq * hier->p : nullptr;
      const int sth = hip_status(asmk::launch_decode_hier(a, *hier, stream), "decode_step_hier");
      if (sth != ASM_OK) return sth;
      continue;
    }
    const hipError_t e = phase == 1   ? asmk::launch_decode_fast_main(a, stream)
                         : phase == 2 ? asmk::launch_decode_fast_merge(a, stream)
                                      : asmk::launch_decode(a, dtype, stream);
    const int st = hip_status(e, "decode_step");
    if (st != ASM_OK) return st;
  }
  return ASM_OK;
}

// ---- scratch of the no-allocation decode entry point -------------------------
// One array per GPU, in the code object, so that the entry point needs no
// allocation.  Host code never uses the array's name as an address: the
// address on the current device comes from hipGetSymbolAddress, once per
// device, and is kept in g_scratch.
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) unsigned char scratch[ASM_NOALLOC_SCRATCH_BYTES];

namespace {

// The scratch address on the device of `stream`, which must be the current
// device.
int noalloc_scratch(hipStream_t stream, void** out) {
  int cur = 0, sdev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(ASM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return fail(ASM_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  if (sdev != cur)
    return fail(ASM_ERR_SHAPE, "the stream belongs to device %d but device %d is current", sdev, cur);
  if (cur < 0 || cur >= kMaxScratchDevices)
    return fail(ASM_ERR_SHAPE, "device %d: the no-allocation entry point serves devices 0..%d", cur,
                kMaxScratchDevices - 1);
  void* p = g_scratch[cur].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[cur].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(ASM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", cur,
                    hipGetErrorString(e));
      g_scratch[cur].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ASM_OK;
}

}  // namespace

extern "C" {

int asm_abi_version(void) { return ASM_ABI_VERSION; }

const char* asm_status_str(int status) {
  switch (status) {
    case ASM_OK: return "ok";
    case ASM_ERR_NULL: return "null pointer";
    case ASM_ERR_SHAPE: return "unsupported shape";
    case ASM_ERR_DTYPE: return "unknown dtype";
    case ASM_ERR_ALIGN: return "misaligned pointer or stride";
    case ASM_ERR_WORKSPACE: return "workspace missing or too small";
    case ASM_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* asm_last_error(void) { return g_err; }

// ---------------------------------------------------------------------------
int asm_centroid_inv_norms(int dtype, int H, int K, int d, const void* C, float* cinv,
                           hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (H < 0 || K < 0) return fail(ASM_ERR_SHAPE, "negative H or K");
  if (int64_t(H) * K > (int64_t(1) << 31) - 1) return fail(ASM_ERR_SHAPE, "H*K too large");
  if (int64_t(H) * K == 0) return ok();
  if (!C || !cinv) return fail(ASM_ERR_NULL, "C and cinv are required");
  ASM_TRY(check_bf16_ptrs(dtype, {C}));
  return hip_status(asmk::launch_inv_norms(dtype, H, K, d, C, cinv, stream), "centroid_inv_norms");
}

// ---------------------------------------------------------------------------
size_t asm_decode_step_ws(int dtype, int B, int Hq, int Hkv, int d, int K, int max_kv_len) {
  if (validate_decode_shape(dtype, B, Hq, Hkv, d, K, max_kv_len) != ASM_OK) return 0;
  // The KV stride decides between the two layouts only at call time: size
  // the workspace for whichever is larger.
  const size_t fast = plan_decode(dtype, B, Hq, Hkv, d, K, max_kv_len, d).total;
  const size_t slow = plan_decode(dtype, B, Hq, Hkv, d, K, max_kv_len, int64_t(1) << 40).total;
  return fast > slow ? fast : slow;
}

int asm_decode_step(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                    const void* q, const void* C, const float* cinv, const float* Abar,
                    const float* LSEbar, const void* Kl, const void* Vl,
                    int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                    const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                    float* out, float* out_lse, int32_t* out_idx,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, out_idx, ws, ws_bytes, stream, nullptr);
}

int asm_decode_step_begin(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                          const void* q, const void* C, const float* cinv, const float* Abar,
                          const float* LSEbar, const void* Kl, const void* Vl,
                          int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                          const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                          float* out, float* out_lse, int32_t* out_idx,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, out_idx, ws, ws_bytes, stream, nullptr, nullptr, false, 1);
}

int asm_decode_step_finish(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                           const void* q, const void* C, const float* cinv, const float* Abar,
                           const float* LSEbar, const void* Kl, const void* Vl,
                           int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                           const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                           float* out, float* out_lse, int32_t* out_idx,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, out_idx, ws, ws_bytes, stream, nullptr, nullptr, false, 2);
}

// ---------------------------------------------------------------------------
int asm_decode_step_noalloc(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                            const void* q, const void* C, const float* cinv, const float* Abar,
                            const float* LSEbar, const void* Kl, const void* Vl,
                            int64_t kv_head_stride, int64_t kv_tok_stride, int64_t kv_capacity,
                            const int32_t* kv_start, const int32_t* kv_len, int max_kv_len,
                            float* out, float* out_lse, int32_t* out_idx, hipStream_t stream) {
  ASM_TRY(check_decode_args(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                            kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len,
                            max_kv_len, out, false));
  // the layout this call will use (the KV stride picks it), not the larger
  // of the two that asm_decode_step_ws reports
  const size_t need = plan_decode(dtype, B, Hq, Hkv, d, K, max_kv_len, kv_tok_stride).total;
  if (need > ASM_NOALLOC_SCRATCH_BYTES)
    return fail(ASM_ERR_WORKSPACE,
                "decode step needs %zu bytes of scratch; asm_decode_step_noalloc holds %zu "
                "(use asm_decode_step with a workspace)",
                need, size_t(ASM_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  ASM_TRY(noalloc_scratch(stream, &ws));
  return decode_impl(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, out_idx, ws, ASM_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

// ---------------------------------------------------------------------------
size_t asm_attend_step_ws(int dtype, int B, int Hq, int Hkv, int d, int max_kv_len) {
  if (validate_decode_shape(dtype, B, Hq, Hkv, d, 1, max_kv_len) != ASM_OK) return 0;
  const DecodePlan p = plan_decode(dtype, B, Hq, Hkv, d, 1, max_kv_len, d, 1);
  return p.fast ? p.total : 0;
}

int asm_attend_step(int dtype, int B, int Hq, int Hkv, int d, float scale, const void* q,
                    const void* Kc, const void* Vc, int64_t kv_head_stride, int64_t kv_tok_stride,
                    int64_t kv_capacity, const int32_t* kv_start, const int32_t* kv_len,
                    int max_kv_len, float* out, float* out_lse, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return decode_impl(dtype, B, Hq, Hkv, d, 1, scale, q, nullptr, nullptr, nullptr, nullptr, Kc, Vc,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, nullptr, ws, ws_bytes, stream, nullptr, nullptr, true);
}

// ---------------------------------------------------------------------------
size_t asm_whiten_fit_ws(int dtype, int H, int N, int d) {
  if (check_dtype(dtype) != ASM_OK || (d != 64 && d != 128) || H < 1 || N < 1) return 0;
  return asmk::whiten_fit_ws_bytes(H, N, d);
}

int asm_whiten_fit(int dtype, int H, int N, int d, const void* X, double ridge, double* mu,
                   double* W, double* resid, void* ws, size_t ws_bytes, hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  if (d != 64 && d != 128) return fail(ASM_ERR_SHAPE, "whitening needs d in {64, 128} (d=%d)", d);
  if (H < 1 || N < 1) return fail(ASM_ERR_SHAPE, "need H, N >= 1 (H=%d, N=%d)", H, N);
  if (int64_t(H) * N > (int64_t(1) << 31) / d) return fail(ASM_ERR_SHAPE, "H*N*d too large");
  if (!(ridge >= 0.0) || ridge == INFINITY) return fail(ASM_ERR_SHAPE, "ridge must be finite and >= 0");
  if (!X || !mu || !W) return fail(ASM_ERR_NULL, "X, mu and W are required");
  ASM_TRY(check_bf16_ptrs(dtype, {X}));
  const size_t need = asmk::whiten_fit_ws_bytes(H, N, d);
  ASM_TRY(check_ws(ws, ws_bytes, need));
  asmk::WhitenFitArgs a{};
  a.H = H; a.N = N; a.d = d; a.nblk = asmk::whiten_blocks(H, N); a.max_iters = 100;
  a.ridge = ridge; a.X = X; a.mu = mu; a.W = W; a.resid = resid;
  char* w = static_cast<char*>(ws);
  a.part_mean = reinterpret_cast<double*>(w);
  w += asmk::align_up(size_t(H) * a.nblk * d * 8, kAlign);
  a.part_cov = reinterpret_cast<double*>(w);
  w += asmk::align_up(size_t(H) * a.nblk * d * d * 8, kAlign);
  a.mats = reinterpret_cast<double*>(w);
  return hip_status(asmk::launch_whiten_fit(a, dtype, stream), "whiten_fit");
}

int asm_whiten_rows(int dtype, int H, int64_t M, int d, const void* Y, int64_t head_stride,
                    int64_t row_stride, const double* mu, const double* W, void* Yw,
                    hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  if (d != 64 && d != 128) return fail(ASM_ERR_SHAPE, "whitening needs d in {64, 128} (d=%d)", d);
  if (H < 1 || M < 0 || head_stride < 0 || row_stride < 0)
    return fail(ASM_ERR_SHAPE, "need H >= 1 and M, strides >= 0");
  if (M == 0) return ok();
  if ((M + 31) / 32 * H * (d / 16) >= (int64_t(1) << 31))
    return fail(ASM_ERR_SHAPE, "too many rows for one launch");
  if (!Y || !Yw || !mu || !W) return fail(ASM_ERR_NULL, "Y, Yw, mu and W are required");
  if (Y == Yw) return fail(ASM_ERR_SHAPE, "Yw must not alias Y");
  if (reinterpret_cast<uintptr_t>(W) % 16 != 0) return fail(ASM_ERR_ALIGN, "W must be 16-byte aligned");
  asmk::WhitenRowsArgs a{};
  a.H = H; a.d = d; a.M = M; a.head_stride = head_stride; a.row_stride = row_stride;
  a.Y = Y; a.Yw = Yw; a.mu = mu; a.W = W;
  return hip_status(asmk::launch_whiten_rows(a, dtype, stream), "whiten_rows");
}

size_t asm_decode_step_whitened_ws(int dtype, int B, int Hq, int Hkv, int d, int K,
                                   int max_kv_len) {
  if (d != 64 && d != 128) return 0;
  const size_t base = asm_decode_step_ws(dtype, B, Hq, Hkv, d, K, max_kv_len);
  if (base == 0) return 0;
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  return asmk::align_up(size_t(B) * Hq * d * esz, kAlign) + base;
}

int asm_decode_step_whitened(int dtype, int B, int Hq, int Hkv, int d, int K, float scale,
                             const void* q, const double* mu, const double* W, const void* Cw,
                             const float* cwinv, const float* Abar, const float* LSEbar,
                             const void* Kl, const void* Vl, int64_t kv_head_stride,
                             int64_t kv_tok_stride, int64_t kv_capacity, const int32_t* kv_start,
                             const int32_t* kv_len, int max_kv_len, float* out, float* out_lse,
                             int32_t* out_idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  if (d != 64 && d != 128) return fail(ASM_ERR_SHAPE, "whitening needs d in {64, 128} (d=%d)", d);
  ASM_TRY(validate_decode_shape(dtype, B, Hq, Hkv, d, K, max_kv_len));
  if (!q || !mu || !W) return fail(ASM_ERR_NULL, "q, mu and W are required");
  ASM_TRY(check_bf16_ptrs(dtype, {q}));
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  const size_t qbytes = asmk::align_up(size_t(B) * Hq * d * esz, kAlign);
  const size_t need = asm_decode_step_whitened_ws(dtype, B, Hq, Hkv, d, K, max_kv_len);
  ASM_TRY(check_ws(ws, ws_bytes, need));
  void* qw = ws;
  // queries [B, Hq, d]: head h row b at h*d + b*Hq*d
  ASM_TRY(asm_whiten_rows(dtype, Hq, B, d, q, d, int64_t(Hq) * d, mu, W, qw, stream));
  return decode_impl(dtype, B, Hq, Hkv, d, K, scale, q, Cw, cwinv, Abar, LSEbar, Kl, Vl,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, out_idx, static_cast<char*>(ws) + qbytes, ws_bytes - qbytes,
                     stream, nullptr, qw);
}

size_t asm_decode_step_hier_ws(int dtype, int B, int Hq, int Hkv, int d, int K, int S, int p,
                               int max_kv_len) {
  if (validate_decode_shape(dtype, B, Hq, Hkv, d, K, max_kv_len) != ASM_OK) return 0;
  if (S < 1 || S > K || p < 1 || p > asmk::kHierMaxProbes) return 0;
  return plan_decode(dtype, B, Hq, Hkv, d, K, max_kv_len, d, p).total;
}

int asm_decode_step_hier(int dtype, int B, int Hq, int Hkv, int d, int K, int S, int p,
                         float scale, const void* q, const void* C, const float* cinv,
                         const void* SC, const float* scinv, const int32_t* offsets,
                         const int32_t* members, const void* Cg, const float* cginv,
                         const float* Abar, const float* LSEbar,
                         const void* Kl, const void* Vl, int64_t kv_head_stride,
                         int64_t kv_tok_stride, int64_t kv_capacity, const int32_t* kv_start,
                         const int32_t* kv_len, int max_kv_len, float* out, float* out_lse,
                         int32_t* out_idx, int32_t* out_probes, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  if (!asmk::hier_fast_path(dtype, d))
    return fail(ASM_ERR_SHAPE, "the hierarchical lookup needs bf16 and d in {64, 128}");
  if (S < 1 || S > K || S > asmk::kHierMaxSupers)
    return fail(ASM_ERR_SHAPE, "need 1 <= S <= min(K, %d) (S=%d, K=%d)", asmk::kHierMaxSupers, S, K);
  if (p < 1 || p > asmk::kHierMaxProbes)
    return fail(ASM_ERR_SHAPE, "need 1 <= p <= %d (p=%d)", asmk::kHierMaxProbes, p);
  if (int64_t(K) * d * 2 >= (int64_t(1) << 31))
    return fail(ASM_ERR_SHAPE, "one head's entry table must stay under 2 GiB (K=%d)", K);
  if (!SC || !scinv || !offsets || !members) return fail(ASM_ERR_NULL, "SC, scinv, offsets and members are required");
  if ((Cg == nullptr) != (cginv == nullptr))
    return fail(ASM_ERR_NULL, "Cg and cginv must both be given or both be NULL");
  ASM_TRY(check_bf16_ptrs(dtype, {SC, Cg}));
  asmk::HierArgs h{};
  h.Hq = Hq; h.K = K; h.S = S; h.d = d; h.p = p;
  h.C = C; h.cinv = cinv; h.SC = SC; h.scinv = scinv; h.offsets = offsets; h.members = members;
  h.Cg = Cg; h.cginv = cginv;
  h.probes_out = out_probes;
  return decode_impl(dtype, B, Hq, Hkv, d, K, scale, q, C, cinv, Abar, LSEbar, Kl, Vl,
                     kv_head_stride, kv_tok_stride, kv_capacity, kv_start, kv_len, max_kv_len,
                     out, out_lse, out_idx, ws, ws_bytes, stream, &h);
}

// ---------------------------------------------------------------------------
size_t asm_build_states_ws(int dtype, int Hq, int Hkv, int N, int L, int d, int chunk) {
  (void)chunk;
  if (check_dtype(dtype) != ASM_OK || check_d(dtype, d) != ASM_OK || Hq < 1 || Hkv < 1 ||
      Hq % Hkv != 0 || N < 0 || L < 0)
    return 0;
  return asmk::states_ws_bytes(dtype, Hq, Hkv, N, L, d);
}

int asm_build_states(int dtype, int Hq, int Hkv, int N, int L, int d, int chunk, float scale,
                     const void* Q, const void* Kp, const void* Vp,
                     float* A_chunks, float* LSE_chunks, float* A, float* LSE, int accumulate,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (Hq < 1 || Hkv < 1 || N < 0 || L < 0 || chunk < 1)
    return fail(ASM_ERR_SHAPE, "need Hq, Hkv, chunk >= 1 and N, L >= 0");
  if (Hq % Hkv != 0) return fail(ASM_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (int64_t(Hq) * N > (int64_t(1) << 30)) return fail(ASM_ERR_SHAPE, "Hq*N too large");
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(ASM_ERR_SHAPE, "scale must be finite");
  if ((A_chunks == nullptr) != (LSE_chunks == nullptr))
    return fail(ASM_ERR_NULL, "A_chunks and LSE_chunks must both be given or both be NULL");
  if (N == 0) return ok();
  if (!Q || !A || !LSE) return fail(ASM_ERR_NULL, "Q, A and LSE are required");
  if (L > 0 && (!Kp || !Vp)) return fail(ASM_ERR_NULL, "Kp and Vp are required when L > 0");
  ASM_TRY(check_bf16_ptrs(dtype, {Q, Kp, Vp}));
  const size_t need = asmk::states_ws_bytes(dtype, Hq, Hkv, N, L, d);
  ASM_TRY(check_ws(ws, ws_bytes, need));
  asmk::StatesArgs a{};
  a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.L = L; a.d = d; a.chunk = chunk;
  a.nc = L > 0 ? int((int64_t(L) + chunk - 1) / chunk) : 0;
  a.scale2 = scale * ASM_LOG2E;
  a.Q = Q; a.Kp = Kp; a.Vp = Vp;
  a.A_chunks = A_chunks; a.LSE_chunks = LSE_chunks; a.A = A; a.LSE = LSE;
  a.accumulate = accumulate ? 1 : 0;
  a.V16 = need > 0 ? ws : nullptr;
  a.v_overflow = need > 0 ? reinterpret_cast<int*>(static_cast<char*>(ws) + asmk::states_v16_bytes(Hkv, L, d))
                          : nullptr;
  return hip_status(asmk::launch_build_states(a, dtype, stream), "build_states");
}

// Streamed prefix: chunk c is staged into slot c % 2 of the workspace on the
// copy stream while the compute stream encodes chunk c - 1; each chunk is
// one asm_build_states call that merges into (A, LSE).
namespace {
size_t stream_slot_bytes(int dtype, int Hkv, int d, int chunk) {
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  return asmk::align_up(size_t(Hkv) * chunk * d * esz, kAlign);
}

struct EventSet {
  hipEvent_t e[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  ~EventSet() {
    for (hipEvent_t x : e)
      if (x) (void)hipEventDestroy(x);
  }
};
}  // namespace

size_t asm_build_states_streamed_ws(int dtype, int Hq, int Hkv, int N, int d, int chunk) {
  if (check_dtype(dtype) != ASM_OK || check_d(dtype, d) != ASM_OK || Hq < 1 || Hkv < 1 ||
      Hq % Hkv != 0 || N < 0 || chunk < 1)
    return 0;
  return 4 * stream_slot_bytes(dtype, Hkv, d, chunk) +
         asmk::align_up(asmk::states_ws_bytes(dtype, Hq, Hkv, N, chunk, d), kAlign);
}

int asm_build_states_streamed(int dtype, int Hq, int Hkv, int N, int L, int d, int chunk,
                              float scale, const void* Q, const void* Kp_host,
                              const void* Vp_host, float* A, float* LSE, int accumulate,
                              void* ws, size_t ws_bytes, hipStream_t stream,
                              hipStream_t copy_stream) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (Hq < 1 || Hkv < 1 || N < 0 || L < 0 || chunk < 1)
    return fail(ASM_ERR_SHAPE, "need Hq, Hkv, chunk >= 1 and N, L >= 0");
  if (Hq % Hkv != 0) return fail(ASM_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (N == 0) return ok();
  if (!Q || !A || !LSE) return fail(ASM_ERR_NULL, "Q, A and LSE are required");
  if (L > 0 && (!Kp_host || !Vp_host)) return fail(ASM_ERR_NULL, "Kp and Vp are required when L > 0");
  const size_t need = asm_build_states_streamed_ws(dtype, Hq, Hkv, N, d, chunk);
  if (need == 0) return fail(ASM_ERR_SHAPE, "unsupported shape");
  ASM_TRY(check_ws(ws, ws_bytes, need));
  if (L == 0) {
    // no prefix: the states of an empty prefix, through the plain entry point
    return asm_build_states(dtype, Hq, Hkv, N, 0, d, chunk, scale, Q, nullptr, nullptr, nullptr,
                            nullptr, A, LSE, accumulate, nullptr, 0, stream);
  }
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  const size_t slot = stream_slot_bytes(dtype, Hkv, d, chunk);
  char* w = static_cast<char*>(ws);
  void* states_ws = w + 4 * slot;
  const size_t states_ws_bytes = ws_bytes - 4 * slot;
  // one stream given (or the same twice): copies and compute share it
  const bool two = copy_stream != stream;
  hipStream_t cs = two ? copy_stream : stream;
  EventSet ev;  // [0] start, [1..2] slot ready, [3..4] slot free
  for (hipEvent_t& e : ev.e) {
    const int st = hip_status(hipEventCreateWithFlags(&e, hipEventDisableTiming), "event create");
    if (st != ASM_OK) return st;
  }
  if (two) {
    // staging may still be read by earlier work on the compute stream
    ASM_TRY(hip_status(hipEventRecord(ev.e[0], stream), "event record"));
    ASM_TRY(hip_status(hipStreamWaitEvent(cs, ev.e[0], 0), "stream wait"));
  }
  const int nc = int((int64_t(L) + chunk - 1) / chunk);
  for (int c = 0; c < nc; ++c) {
    const int sl = c & 1;
    const int64_t t0 = int64_t(c) * chunk;
    const int len = int(L - t0 < chunk ? L - t0 : chunk);
    char* kd = w + (2 * sl) * slot;
    char* vd = w + (2 * sl + 1) * slot;
    if (two && c >= 2) ASM_TRY(hip_status(hipStreamWaitEvent(cs, ev.e[3 + sl], 0), "stream wait"));
    // [Hkv, L, d] host rows t0 .. t0+len of every kv head -> [Hkv, len, d]
    const size_t row = size_t(len) * d * esz, spitch = size_t(L) * d * esz;
    ASM_TRY(hip_status(hipMemcpy2DAsync(kd, row, static_cast<const char*>(Kp_host) + t0 * d * esz,
                                        spitch, row, size_t(Hkv), hipMemcpyHostToDevice, cs),
                       "copy K"));
    ASM_TRY(hip_status(hipMemcpy2DAsync(vd, row, static_cast<const char*>(Vp_host) + t0 * d * esz,
                                        spitch, row, size_t(Hkv), hipMemcpyHostToDevice, cs),
                       "copy V"));
    if (two) {
      ASM_TRY(hip_status(hipEventRecord(ev.e[1 + sl], cs), "event record"));
      ASM_TRY(hip_status(hipStreamWaitEvent(stream, ev.e[1 + sl], 0), "stream wait"));
    }
    ASM_TRY(asm_build_states(dtype, Hq, Hkv, N, len, d, len, scale, Q, kd, vd, nullptr, nullptr,
                             A, LSE, (c > 0 || accumulate) ? 1 : 0, states_ws, states_ws_bytes,
                             stream));
    if (two) ASM_TRY(hip_status(hipEventRecord(ev.e[3 + sl], stream), "event record"));
  }
  return ok();
}

// ---------------------------------------------------------------------------
size_t asm_kmeans_assign_ws(int dtype, int H, int N, int K, int d) {
  (void)dtype; (void)H; (void)N; (void)K; (void)d;
  return 0;
}

int asm_kmeans_assign(int dtype, int H, int N, int K, int d, const void* X, const void* C,
                      const float* cinv, int32_t* idx, float* best,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws; (void)ws_bytes;
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (H < 0 || N < 0 || K < 1) return fail(ASM_ERR_SHAPE, "need H, N >= 0 and K >= 1");
  if (int64_t(H) * N > (int64_t(1) << 30) || int64_t(H) * K > (int64_t(1) << 30))
    return fail(ASM_ERR_SHAPE, "H*N or H*K too large");
  if (int64_t(H) * N == 0) return ok();
  if (!X || !C || !cinv || !idx) return fail(ASM_ERR_NULL, "X, C, cinv and idx are required");
  ASM_TRY(check_bf16_ptrs(dtype, {X, C}));
  asmk::AssignArgs a{};
  a.H = H; a.N = N; a.K = K; a.d = d;
  a.X = X; a.C = C; a.cinv = cinv; a.idx = idx; a.best = best;
  return hip_status(asmk::launch_assign(a, dtype, stream), "kmeans_assign");
}

// ---------------------------------------------------------------------------
static bool aggregate_lds_sort(int K) { return K <= asmk::kAggLdsMaxK; }

static size_t aggregate_ws_bytes(int H, int N, int K) {
  size_t off = asmk::align_up(size_t(H) * (K + 1) * sizeof(int32_t), kAlign);
  off += asmk::align_up(size_t(H) * K * sizeof(int32_t), kAlign);
  off += asmk::align_up(size_t(H) * N * sizeof(int32_t), kAlign);
  if (aggregate_lds_sort(K))
    off += asmk::align_up(size_t(H) * K * asmk::agg_chunks(N) * sizeof(int32_t), kAlign);
  return off;
}

size_t asm_aggregate_ws(int dtype, int H, int N, int K, int d) {
  if (check_dtype(dtype) != ASM_OK || check_d(dtype, d) != ASM_OK || H < 0 || N < 0 || K < 1) return 0;
  return aggregate_ws_bytes(H, N, K);
}

int asm_aggregate(int dtype, int H, int N, int K, int d, const void* X, const int32_t* idx,
                  const float* A, const float* LSE, void* C, float* cinv, int32_t* count,
                  float* Abar, float* LSEbar, void* ws, size_t ws_bytes, hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (H < 0 || N < 0 || K < 1) return fail(ASM_ERR_SHAPE, "need H, N >= 0 and K >= 1");
  if (int64_t(H) * N > (int64_t(1) << 30) || int64_t(H) * K > (int64_t(1) << 30))
    return fail(ASM_ERR_SHAPE, "H*N or H*K too large");
  if (H == 0) return ok();
  if (!C || !cinv || !count) return fail(ASM_ERR_NULL, "C, cinv and count are required");
  if (N > 0 && (!X || !idx)) return fail(ASM_ERR_NULL, "X and idx are required when N > 0");
  if ((Abar == nullptr) != (LSEbar == nullptr))
    return fail(ASM_ERR_NULL, "Abar and LSEbar must both be given or both be NULL");
  if (Abar && N > 0 && (!A || !LSE)) return fail(ASM_ERR_NULL, "A and LSE are required with Abar");
  ASM_TRY(check_bf16_ptrs(dtype, {X, C}));
  const size_t need = aggregate_ws_bytes(H, N, K);
  ASM_TRY(check_ws(ws, ws_bytes, need));
  asmk::AggregateArgs a{};
  a.H = H; a.N = N; a.K = K; a.d = d;
  a.X = X; a.idx = idx; a.A = A; a.LSE = LSE; a.C = C; a.cinv = cinv; a.count = count;
  a.Abar = Abar; a.LSEbar = LSEbar;
  char* w = static_cast<char*>(ws);
  size_t off = 0;
  a.offsets = reinterpret_cast<int32_t*>(w + off);
  off += asmk::align_up(size_t(H) * (K + 1) * sizeof(int32_t), kAlign);
  a.cursor = reinterpret_cast<int32_t*>(w + off);
  off += asmk::align_up(size_t(H) * K * sizeof(int32_t), kAlign);
  a.perm = reinterpret_cast<int32_t*>(w + off);
  off += asmk::align_up(size_t(H) * N * sizeof(int32_t), kAlign);
  a.part = aggregate_lds_sort(K) ? reinterpret_cast<int32_t*>(w + off) : nullptr;
  return hip_status(asmk::launch_aggregate(a, dtype, stream), "aggregate");
}

// ---------------------------------------------------------------------------
size_t asm_build_memory_ws(int dtype, int H, int N, int K, int d) {
  const size_t a = asm_kmeans_assign_ws(dtype, H, N, K, d);
  const size_t g = asm_aggregate_ws(dtype, H, N, K, d);
  if (check_dtype(dtype) != ASM_OK || check_d(dtype, d) != ASM_OK || H < 1 || K < 1 || N < K)
    return 0;
  return a > g ? a : g;
}

int asm_build_memory(int dtype, int H, int N, int K, int d, int iters, const void* X,
                     const float* A, const float* LSE, void* C, float* cinv, float* Abar,
                     float* LSEbar, int32_t* count, int32_t* idx, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (H < 1 || K < 1 || N < K || iters < 1)
    return fail(ASM_ERR_SHAPE, "need H, K >= 1, N >= K and iters >= 1 (H=%d N=%d K=%d iters=%d)",
                H, N, K, iters);
  if (!X || !C || !cinv || !count || !idx)
    return fail(ASM_ERR_NULL, "X, C, cinv, count and idx are required");
  if ((A == nullptr) != (LSE == nullptr) || (Abar == nullptr) != (A == nullptr) ||
      (LSEbar == nullptr) != (A == nullptr))
    return fail(ASM_ERR_NULL, "A, LSE, Abar and LSEbar must all be given or all be NULL");
  ASM_TRY(check_bf16_ptrs(dtype, {X, C}));
  ASM_TRY(check_ws(ws, ws_bytes, asm_build_memory_ws(dtype, H, N, K, d)));
  // first-K initialisation: C[h] = X[h, :K]
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  ASM_TRY(hip_status(hipMemcpy2DAsync(C, size_t(K) * d * esz, X, size_t(N) * d * esz,
                                      size_t(K) * d * esz, size_t(H), hipMemcpyDeviceToDevice,
                                      stream),
                     "copy initial centroids"));
  ASM_TRY(asm_centroid_inv_norms(dtype, H, K, d, C, cinv, stream));
  for (int t = 0; t < iters; ++t) {
    const bool last = t == iters - 1;
    ASM_TRY(asm_kmeans_assign(dtype, H, N, K, d, X, C, cinv, idx, nullptr, ws, ws_bytes, stream));
    ASM_TRY(asm_aggregate(dtype, H, N, K, d, X, idx, last ? A : nullptr, last ? LSE : nullptr, C,
                          cinv, count, last ? Abar : nullptr, last ? LSEbar : nullptr, ws, ws_bytes,
                          stream));
  }
  return ok();
}

// ---------------------------------------------------------------------------
static size_t build_index_ws_bytes(int H, int K, int S) {
  size_t off = asmk::align_up(size_t(H) * K * sizeof(int32_t), kAlign);  // entry -> super
  off += asmk::align_up(size_t(H) * S * sizeof(int32_t), kAlign);        // scatter cursors
  return off;
}

int asm_index_group_rows(int dtype, int H, int K, int d, const void* C, const float* cinv,
                         const int32_t* members, void* Cg, float* cginv, hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  if (d != 64 && d != 128) return fail(ASM_ERR_SHAPE, "need d in {64, 128} (d=%d)", d);
  if (H < 1 || K < 1) return fail(ASM_ERR_SHAPE, "need H, K >= 1 (H=%d, K=%d)", H, K);
  if (!C || !cinv || !members || !Cg || !cginv)
    return fail(ASM_ERR_NULL, "C, cinv, members, Cg and cginv are required");
  if (!aligned16(C) || !aligned16(Cg)) return fail(ASM_ERR_ALIGN, "C and Cg must be 16-byte aligned");
  const size_t row_bytes = size_t(d) * (dtype == ASM_BF16 ? 2 : 4);
  const char* c0 = static_cast<const char*>(C);
  const char* g0 = static_cast<const char*>(Cg);
  const size_t bytes = size_t(H) * K * row_bytes;
  if (g0 < c0 + bytes && c0 < g0 + bytes) return fail(ASM_ERR_SHAPE, "Cg must not overlap C");
  return hip_status(asmk::launch_index_group_rows(dtype, H, K, d, C, cinv, members, Cg, cginv, stream),
                    "index_group_rows");
}

size_t asm_build_index_ws(int dtype, int H, int K, int S, int d) {
  if (check_dtype(dtype) != ASM_OK || check_d(dtype, d) != ASM_OK || H < 0 || K < 1 || S < 1 || S > K)
    return 0;
  return build_index_ws_bytes(H, K, S);
}

int asm_build_index(int dtype, int H, int K, int S, int d, int iters, const void* C, void* SC,
                    float* scinv, int32_t* counts, int32_t* offsets, int32_t* members, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  ASM_TRY(check_dtype(dtype));
  ASM_TRY(check_d(dtype, d));
  if (H < 0 || K < 1 || S < 1 || S > K || iters < 1)
    return fail(ASM_ERR_SHAPE, "need H >= 0, 1 <= S <= K and iters >= 1 (S=%d K=%d iters=%d)", S, K, iters);
  if (int64_t(H) * K > (int64_t(1) << 30)) return fail(ASM_ERR_SHAPE, "H*K too large");
  if (H == 0) return ok();
  if (!C || !SC || !scinv || !counts || !offsets || !members)
    return fail(ASM_ERR_NULL, "C, SC, scinv, counts, offsets and members are required");
  ASM_TRY(check_bf16_ptrs(dtype, {C, SC}));
  ASM_TRY(check_ws(ws, ws_bytes, build_index_ws_bytes(H, K, S)));
  char* w = static_cast<char*>(ws);
  int32_t* e2s = reinterpret_cast<int32_t*>(w);
  int32_t* cursor = reinterpret_cast<int32_t*>(w + asmk::align_up(size_t(H) * K * sizeof(int32_t), kAlign));
  const size_t esz = dtype == ASM_BF16 ? 2 : 4;
  // first-S initialisation: the first S entries of every head
  int st = hip_status(hipMemcpy2DAsync(SC, size_t(S) * d * esz, C, size_t(K) * d * esz,
                                       size_t(S) * d * esz, size_t(H), hipMemcpyDeviceToDevice, stream),
                      "build_index");
  if (st != ASM_OK) return st;
  st = hip_status(asmk::launch_inv_norms(dtype, H, S, d, SC, scinv, stream), "build_index");
  if (st != ASM_OK) return st;
  for (int it = 0; it < iters; ++it) {
    asmk::AssignArgs as{};
    as.H = H; as.N = K; as.K = S; as.d = d;
    as.X = C; as.C = SC; as.cinv = scinv; as.idx = e2s; as.best = nullptr;
    st = hip_status(asmk::launch_assign(as, dtype, stream), "build_index");
    if (st != ASM_OK) return st;
    // mean step; its counting sort leaves the member lists of this partition
    asmk::AggregateArgs ag{};
    ag.H = H; ag.N = K; ag.K = S; ag.d = d;
    ag.X = C; ag.idx = e2s; ag.C = SC; ag.cinv = scinv; ag.count = counts;
    ag.offsets = offsets; ag.cursor = cursor; ag.perm = members;
    st = hip_status(asmk::launch_aggregate(ag, dtype, stream), "build_index");
    if (st != ASM_OK) return st;
  }
  return ASM_OK;
}

}  // extern "C"

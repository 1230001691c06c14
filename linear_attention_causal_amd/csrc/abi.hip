// C ABI of libgdn: argument validation (fail closed, before any enqueue) and
// dispatch to the gfx950 kernels.  Declarations and semantics: include/gdn.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long long channels(const gdn_geometry& g) {
  return 2LL * g.num_k_heads * g.head_k_dim + (long long)g.num_v_heads * g.head_v_dim;
}

int check_geometry(const gdn_geometry* g) {
  if (!g) return fail(GDN_E_NULL, "geometry is NULL");
  if (g->num_k_heads <= 0 || g->num_v_heads <= 0 || g->head_k_dim <= 0 ||
      g->head_v_dim <= 0 || g->conv_kernel <= 0)
    return fail(GDN_E_SHAPE, "geometry dimensions must be positive");
  if (g->num_v_heads % g->num_k_heads != 0)
    return fail(GDN_E_HEADS, "num_v_heads (%d) is not a multiple of num_k_heads (%d)",
                g->num_v_heads, g->num_k_heads);
  if (g->head_k_dim != g->head_v_dim ||
      (g->head_k_dim != 32 && g->head_k_dim != 64 && g->head_k_dim != 128))
    return fail(GDN_E_UNSUPPORTED, "compiled for head_k_dim == head_v_dim in {32, 64, 128}");
  if (g->conv_kernel < 2 || g->conv_kernel > 4)
    return fail(GDN_E_UNSUPPORTED, "compiled for conv_kernel in 2..4");
  if (g->act_dtype != GDN_F32 && g->act_dtype != GDN_BF16)
    return fail(GDN_E_UNSUPPORTED, "act_dtype must be GDN_F32 or GDN_BF16");
  if (!(g->l2norm_eps >= 0.f) || !(g->rmsnorm_eps >= 0.f))
    return fail(GDN_E_SHAPE, "epsilons must be non-negative");
  if ((long long)g->num_v_heads * g->head_v_dim * g->head_k_dim > (1LL << 28))
    return fail(GDN_E_SHAPE, "per-slot state too large");
  return GDN_OK;
}

int check_weights(const gdn_layer_weights* w) {
  if (!w) return fail(GDN_E_NULL, "weights is NULL");
  if (!w->conv_weight || !w->A_log || !w->dt_bias || !w->norm_weight)
    return fail(GDN_E_NULL, "a weight pointer is NULL");
  if (!aligned16(w->conv_weight) || !aligned16(w->norm_weight))
    return fail(GDN_E_ALIGN, "conv_weight and norm_weight must be 16-byte aligned");
  return GDN_OK;
}

int check_pool(const gdn_state_pool* p, bool need_rec, bool need_conv) {
  if (!p) return fail(GDN_E_NULL, "state pool is NULL");
  if (p->num_slots <= 0) return fail(GDN_E_SHAPE, "num_slots must be positive");
  if ((need_rec && !p->recurrent) || (need_conv && !p->conv))
    return fail(GDN_E_NULL, "state pool pointer is NULL");
  if ((need_rec && !aligned16(p->recurrent)) || (need_conv && !aligned16(p->conv)))
    return fail(GDN_E_ALIGN, "state pools must be 16-byte aligned");
  return GDN_OK;
}

// Host copy of per-row slots: each in [0, num_slots) or negative (padding);
// non-negative entries distinct.
int check_slots_host(const int32_t* s, int n, int num_slots) {
  if (!s) return GDN_OK;
  std::vector<int32_t> live;
  live.reserve(n);
  for (int i = 0; i < n; ++i) {
    if (s[i] >= num_slots)
      return fail(GDN_E_SLOT, "slot_idx[%d] = %d is outside [0, %d)", i, s[i], num_slots);
    if (s[i] >= 0) live.push_back(s[i]);
  }
  std::sort(live.begin(), live.end());
  for (size_t i = 1; i < live.size(); ++i)
    if (live[i] == live[i - 1]) return fail(GDN_E_SLOT, "slot %d named twice", live[i]);
  return GDN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(GDN_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define GDN_TRY(expr)          \
  do {                         \
    const int rc_ = (expr);    \
    if (rc_ != GDN_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_last_error(void) { return g_last_error; }

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_E_NULL: return "null pointer";
    case GDN_E_SHAPE: return "bad size";
    case GDN_E_HEADS: return "num_v_heads not a multiple of num_k_heads";
    case GDN_E_UNSUPPORTED: return "unsupported geometry or dtype";
    case GDN_E_SLOT: return "slot index out of range or duplicated";
    case GDN_E_OVERLAP: return "compaction sources and destinations overlap";
    case GDN_E_SEQLENS: return "malformed cu_seqlens";
    case GDN_E_SCRATCH: return "scratch missing or too small";
    case GDN_E_HIP: return "HIP runtime error";
    case GDN_E_ALIGN: return "pointer not 16-byte aligned";
    default: return "unknown status";
  }
}

int gdn_slot_bytes(const gdn_geometry* geom, size_t* recurrent_bytes, size_t* conv_bytes) {
  GDN_TRY(check_geometry(geom));
  if (!recurrent_bytes || !conv_bytes) return fail(GDN_E_NULL, "output pointer is NULL");
  *recurrent_bytes = (size_t)geom->num_v_heads * geom->head_k_dim * geom->head_v_dim * 4;
  *conv_bytes = (size_t)geom->conv_kernel * channels(*geom) *
                (geom->act_dtype == GDN_BF16 ? 2 : 4);
  return ok();
}

int gdn_prefill_scratch_bytes(const gdn_geometry* geom, int32_t total_tokens,
                              int32_t num_seqs, size_t* bytes) {
  GDN_TRY(check_geometry(geom));
  if (!bytes) return fail(GDN_E_NULL, "output pointer is NULL");
  if (total_tokens < 0 || num_seqs < 0) return fail(GDN_E_SHAPE, "negative size");
  *bytes = gdn::prefill_scratch_bytes(*geom, total_tokens, num_seqs);
  return ok();
}

int gdn_conv_update(const gdn_geometry* geom, const gdn_layer_weights* w,
                    const gdn_state_pool* pool, const int32_t* slot_idx,
                    const int32_t* slot_idx_host, int32_t B, const void* qkv_in,
                    float* qkv_out, void* stream) {
  GDN_TRY(check_geometry(geom));
  GDN_TRY(check_weights(w));
  GDN_TRY(check_pool(pool, false, true));
  if (B < 0 || B > 65535) return fail(GDN_E_SHAPE, "B = %d outside [0, 65535]", B);
  if (B == 0) return ok();
  if (!slot_idx || !qkv_in || !qkv_out) return fail(GDN_E_NULL, "a device array is NULL");
  if (!aligned16(qkv_in) || !aligned16(qkv_out))
    return fail(GDN_E_ALIGN, "qkv_in and qkv_out must be 16-byte aligned");
  GDN_TRY(check_slots_host(slot_idx_host, B, pool->num_slots));
  return hip_status(gdn::launch_conv_update(*geom, *w, *pool, slot_idx, B, qkv_in, qkv_out,
                                            static_cast<hipStream_t>(stream)),
                    "gdn_conv_update launch");
}

int gdn_decode_batch(const gdn_geometry* geom, const gdn_layer_weights* w,
                     const gdn_state_pool* pool, const int32_t* slot_idx,
                     const int32_t* slot_idx_host, int32_t B, const float* qkv,
                     const void* z, const void* a, const void* b, void* y, float* o_raw,
                     void* stream) {
  GDN_TRY(check_geometry(geom));
  GDN_TRY(check_weights(w));
  GDN_TRY(check_pool(pool, true, false));
  if (B < 0) return fail(GDN_E_SHAPE, "B = %d is negative", B);
  if ((long long)B * geom->num_v_heads > 0x7fffffffLL) return fail(GDN_E_SHAPE, "B too large");
  if (B == 0) return ok();
  if (!slot_idx || !qkv || !z || !a || !b || !y) return fail(GDN_E_NULL, "a device array is NULL");
  if (!aligned16(qkv) || !aligned16(z) || !aligned16(y) || (o_raw && !aligned16(o_raw)))
    return fail(GDN_E_ALIGN, "qkv, z, y, o_raw must be 16-byte aligned");
  GDN_TRY(check_slots_host(slot_idx_host, B, pool->num_slots));
  return hip_status(gdn::launch_decode(*geom, *w, *pool, slot_idx, B, qkv, z, a, b, y, o_raw,
                                       static_cast<hipStream_t>(stream)),
                    "gdn_decode_batch launch");
}

int gdn_decode_workspace_bytes(const gdn_geometry* geom, int32_t B, size_t* bytes) {
  GDN_TRY(check_geometry(geom));
  if (!bytes) return fail(GDN_E_NULL, "output pointer is NULL");
  if (B < 0) return fail(GDN_E_SHAPE, "B = %d is negative", B);
  if ((long long)B * geom->num_v_heads > (1LL << 30)) return fail(GDN_E_SHAPE, "B too large");
  *bytes = gdn::decode_workspace_bytes(*geom, B);
  return ok();
}

int gdn_decode_step(const gdn_geometry* geom, const gdn_layer_weights* w,
                    const gdn_state_pool* pool, const int32_t* slot_idx,
                    const int32_t* slot_idx_host, int32_t B, const void* qkv_in, const void* z,
                    const void* a, const void* b, void* y, float* o_raw, void* workspace,
                    size_t workspace_bytes, void* stream) {
  GDN_TRY(check_geometry(geom));
  GDN_TRY(check_weights(w));
  GDN_TRY(check_pool(pool, true, true));
  if (B < 0) return fail(GDN_E_SHAPE, "B = %d is negative", B);
  if ((long long)B * geom->num_v_heads > (1LL << 30)) return fail(GDN_E_SHAPE, "B too large");
  if (B == 0) return ok();
  if (!slot_idx || !qkv_in || !z || !a || !b || !y)
    return fail(GDN_E_NULL, "a device array is NULL");
  if (!aligned16(qkv_in) || !aligned16(z) || !aligned16(y) || (o_raw && !aligned16(o_raw)))
    return fail(GDN_E_ALIGN, "qkv_in, z, y, o_raw must be 16-byte aligned");
  const size_t need = gdn::decode_workspace_bytes(*geom, B);
  if (!workspace || workspace_bytes < need)
    return fail(GDN_E_SCRATCH, "workspace needs %zu bytes for %d rows, got %zu", need, B,
                workspace ? workspace_bytes : (size_t)0);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GDN_E_ALIGN, "workspace must be 256-byte aligned");
  GDN_TRY(check_slots_host(slot_idx_host, B, pool->num_slots));
  return hip_status(gdn::launch_decode_step(*geom, *w, *pool, slot_idx, B, qkv_in, z, a, b, y,
                                            o_raw, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "gdn_decode_step launch");
}

int gdn_decode_step_noalloc(const gdn_geometry* geom, const gdn_layer_weights* w,
                            const gdn_state_pool* pool, const int32_t* slot_idx,
                            const int32_t* slot_idx_host, int32_t B, const void* qkv_in,
                            const void* z, const void* a, const void* b, void* y,
                            float* o_raw, void* stream) {
  GDN_TRY(check_geometry(geom));
  GDN_TRY(check_weights(w));
  GDN_TRY(check_pool(pool, true, true));
  if (B < 0) return fail(GDN_E_SHAPE, "B = %d is negative", B);
  if ((long long)B * geom->num_v_heads > (1LL << 30)) return fail(GDN_E_SHAPE, "B too large");
  if (B == 0) return ok();
  if (!slot_idx || !qkv_in || !z || !a || !b || !y)
    return fail(GDN_E_NULL, "a device array is NULL");
  if (!aligned16(qkv_in) || !aligned16(z) || !aligned16(y) || (o_raw && !aligned16(o_raw)))
    return fail(GDN_E_ALIGN, "qkv_in, z, y, o_raw must be 16-byte aligned");
  const size_t need = gdn::decode_workspace_bytes(*geom, B);
  if (need > gdn::kStaticScratchBytes)
    return fail(GDN_E_SCRATCH,
                "gdn_decode_step_noalloc: %d rows need %zu bytes of workspace, more than the "
                "%zu bytes the library holds; use gdn_decode_step with a workspace",
                B, need, gdn::kStaticScratchBytes);
  GDN_TRY(check_slots_host(slot_idx_host, B, pool->num_slots));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int rc = hip_status(gdn::static_scratch(&ws, st), "gdn_decode_step_noalloc scratch");
  if (rc != GDN_OK) return rc;
  return hip_status(gdn::launch_decode_step(*geom, *w, *pool, slot_idx, B, qkv_in, z, a, b, y,
                                            o_raw, ws, st),
                    "gdn_decode_step_noalloc launch");
}

int gdn_prefill_chunked(const gdn_geometry* geom, const gdn_layer_weights* w,
                        const gdn_state_pool* pool, const int32_t* cu_seqlens_host,
                        const int32_t* cu_seqlens_dev, const int32_t* slot_idx,
                        const int32_t* slot_idx_host, const uint8_t* has_init, int32_t N,
                        const void* qkv_in, const void* z, const void* a, const void* b,
                        void* y, float* o_raw, void* scratch, size_t scratch_bytes,
                        void* stream) {
  GDN_TRY(check_geometry(geom));
  GDN_TRY(check_weights(w));
  GDN_TRY(check_pool(pool, true, true));
  if (N < 0 || N > 65535) return fail(GDN_E_SHAPE, "N = %d outside [0, 65535]", N);
  if (N == 0) return ok();
  if (!cu_seqlens_host || !cu_seqlens_dev || !slot_idx)
    return fail(GDN_E_NULL, "cu_seqlens or slot_idx is NULL");
  if (cu_seqlens_host[0] != 0) return fail(GDN_E_SEQLENS, "cu_seqlens[0] must be 0");
  int max_len = 0;
  for (int i = 0; i < N; ++i) {
    const int len = cu_seqlens_host[i + 1] - cu_seqlens_host[i];
    if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
      return fail(GDN_E_SEQLENS, "cu_seqlens decreases at %d", i);
    max_len = std::max(max_len, len);
  }
  const long long T = cu_seqlens_host[N];
  // per-chunk launches have one workgroup of 256 threads per (chunk, V-head)
  // along x: keep their work-item counts within a dispatch's 32-bit size
  const long long chunks_x = N <= 64 ? (T + 63) / 64 + N : (max_len + 63) / 64;
  if ((chunks_x + 8) * geom->num_v_heads * 256 >= (1LL << 32))
    return fail(GDN_E_SHAPE, "too many tokens for one call (%lld chunks x %d V-heads)", chunks_x,
                geom->num_v_heads);
  GDN_TRY(check_slots_host(slot_idx_host, N, pool->num_slots));
  if (T > 0) {
    if (!qkv_in || !z || !a || !b || !y) return fail(GDN_E_NULL, "a device array is NULL");
    if (!aligned16(qkv_in) || !aligned16(z) || !aligned16(y) || (o_raw && !aligned16(o_raw)))
      return fail(GDN_E_ALIGN, "qkv_in, z, y, o_raw must be 16-byte aligned");
    const size_t need = gdn::prefill_scratch_bytes(*geom, T, N);
    if (!scratch || scratch_bytes < need)
      return fail(GDN_E_SCRATCH, "scratch needs %zu bytes, got %zu", need,
                  scratch ? scratch_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(scratch) & 255u) != 0)
      return fail(GDN_E_ALIGN, "scratch must be 256-byte aligned");
  }
  return hip_status(gdn::launch_prefill(*geom, *w, *pool, cu_seqlens_dev, cu_seqlens_host,
                                        max_len, T, slot_idx,
                                        has_init, N, qkv_in, z, a, b, y, o_raw, scratch,
                                        static_cast<hipStream_t>(stream)),
                    "gdn_prefill_chunked launch");
}

int gdn_check_slots(const int32_t* slot_idx, int32_t B, int32_t num_slots, int32_t* result,
                    void* stream) {
  if (B < 0 || B > (1 << 20)) return fail(GDN_E_SHAPE, "B = %d outside [0, 2^20]", B);
  if (num_slots <= 0) return fail(GDN_E_SHAPE, "num_slots must be positive");
  if (!result || (B > 0 && !slot_idx)) return fail(GDN_E_NULL, "slot_idx or result is NULL");
  if (reinterpret_cast<uintptr_t>(result) & 3u)
    return fail(GDN_E_ALIGN, "result must be 4-byte aligned");
  return hip_status(gdn::launch_check_slots(slot_idx, B, num_slots, result,
                                            static_cast<hipStream_t>(stream)),
                    "gdn_check_slots launch");
}

int gdn_state_compact(const gdn_geometry* geom, const gdn_state_pool* pools, int32_t L,
                      const int32_t* src_host, const int32_t* dst_host,
                      const int32_t* src_dev, const int32_t* dst_dev, int32_t n,
                      void* stream) {
  GDN_TRY(check_geometry(geom));
  if (L < 0 || n < 0 || n > 65535) return fail(GDN_E_SHAPE, "L or n out of range");
  if (L == 0 || n == 0) return ok();
  if (!pools) return fail(GDN_E_NULL, "pools is NULL");
  if (!src_host || !dst_host || !src_dev || !dst_dev)
    return fail(GDN_E_NULL, "src/dst arrays are NULL");
  const int P = pools[0].num_slots;
  for (int l = 0; l < L; ++l) {
    GDN_TRY(check_pool(&pools[l], true, true));
    if (pools[l].num_slots != P) return fail(GDN_E_SHAPE, "pools differ in num_slots");
  }
  std::vector<char> role(P, 0);  // 1 = source, 2 = destination
  for (int i = 0; i < n; ++i) {
    const int s = src_host[i], d = dst_host[i];
    if (s < 0 || s >= P || d < 0 || d >= P)
      return fail(GDN_E_SLOT, "pair %d (%d -> %d) outside [0, %d)", i, s, d, P);
    if (role[d] == 2) return fail(GDN_E_SLOT, "destination %d named twice", d);
    role[d] = 2;
  }
  for (int i = 0; i < n; ++i)
    if (role[src_host[i]] == 2)
      return fail(GDN_E_OVERLAP, "slot %d is both a source and a destination", src_host[i]);
  return hip_status(gdn::launch_compact(*geom, pools, L, src_dev, dst_dev, n,
                                        static_cast<hipStream_t>(stream)),
                    "gdn_state_compact launch");
}

int gdn_linear(const void* x, int32_t M, int32_t K, int32_t ldx, const gdn_linear_out* outs,
               int32_t count, void* stream) {
  if (M < 0 || K <= 0 || K % 8 != 0 || ldx < K || ldx % 8 != 0)
    return fail(GDN_E_SHAPE, "need M >= 0, K > 0, K and ldx multiples of 8, ldx >= K");
  if (count < 1 || count > gdn::kMaxLinearOuts)
    return fail(GDN_E_SHAPE, "count must be in 1..%d", gdn::kMaxLinearOuts);
  if (!outs) return fail(GDN_E_NULL, "outs is NULL");
  if (M > 65535 * 16) return fail(GDN_E_SHAPE, "M too large");
  if (M == 0) return ok();
  if (!x) return fail(GDN_E_NULL, "x is NULL");
  if (!aligned16(x)) return fail(GDN_E_ALIGN, "x must be 16-byte aligned");
  // byte ranges [lo, hi) that outputs must not touch
  struct Range { uintptr_t lo, hi; };
  const auto range = [](const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
  };
  const auto overlap = [](Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; };
  std::vector<Range> reads{range(x, ((size_t)(M - 1) * ldx + K) * 2)}, writes;
  gdn::LinearOut lo[gdn::kMaxLinearOuts];
  long long tiles = 0;
  for (int i = 0; i < count; ++i) {
    const gdn_linear_out& o = outs[i];
    if (!o.weight || !o.out) return fail(GDN_E_NULL, "output %d has a NULL pointer", i);
    if (o.N <= 0 || o.ldy < o.N) return fail(GDN_E_SHAPE, "output %d: need 0 < N <= ldy", i);
    if (!aligned16(o.weight)) return fail(GDN_E_ALIGN, "weight %d must be 16-byte aligned", i);
    if (reinterpret_cast<uintptr_t>(o.out) & 1u)
      return fail(GDN_E_ALIGN, "output %d must be 2-byte aligned", i);
    reads.push_back(range(o.weight, (size_t)o.N * K * 2));
    writes.push_back(range(o.out, ((size_t)(M - 1) * o.ldy + o.N) * 2));
    tiles += (o.N + 15) / 16;
    lo[i] = gdn::LinearOut{static_cast<const __bf16*>(o.weight), static_cast<__bf16*>(o.out),
                           o.N, o.ldy, 0};
  }
  if (tiles > 0x7fffffff) return fail(GDN_E_SHAPE, "too many output columns");
  for (size_t i = 0; i < writes.size(); ++i) {
    for (const Range& r : reads)
      if (overlap(writes[i], r)) return fail(GDN_E_OVERLAP, "output %zu overlaps an input", i);
    for (size_t j = i + 1; j < writes.size(); ++j)
      if (overlap(writes[i], writes[j]))
        return fail(GDN_E_OVERLAP, "outputs %zu and %zu overlap", i, j);
  }
  return hip_status(gdn::launch_linear(x, M, K, ldx, lo, count, static_cast<hipStream_t>(stream)),
                    "gdn_linear launch");
}

}  // extern "C"

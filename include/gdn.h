/*
 * gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet layer core.
 *
 * The layer is the linear-attention ("GDR", gated delta rule) block of
 * Qwen3.5 / Qwen3-Next as the pages describe it:
 *   - fused [q|k|v] projection output fed through a depthwise causal conv1d
 *     (pegainfer PR #1003 "shard linear-attention/GDR state per TP rank",
 *     PR body, weight_loader bullet; cortex commit 95dc874 "TP-aware
 *     Qwen3-Next", Architecture pieces, TpQwen3_5GatedDeltaNet);
 *   - l2-normalised q, k; K-heads repeat_interleave'd onto V-heads
 *     (cortex commit 95dc874, Helpers in arch/qwen3_5/linear_attn.rs and
 *     "Reuses unchanged");
 *   - softplus gating from A_log / dt_bias and in_proj_a / in_proj_b
 *     (cortex commit 95dc874, TpQwen3_5GatedDeltaNet);
 *   - the delta-rule state update per V-head, state never all-reduced
 *     (pegainfer PR #1003, PR body, last line; cortex commit 95dc874,
 *     TpQwen3_5GatedDeltaNet): with g = -exp(A_log) softplus(a + dt_bias),
 *     beta = sigmoid(b),
 *         S_t = e^g S_{t-1} + beta k (v - e^g S_{t-1}^T k)^T,   o = S_t^T q
 *     (the gated delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta
 *     Networks", ICLR 2025), with q scaled by 1/sqrt(dk);
 *   - gated RMSNorm at the local V-heads with a head-shared weight,
 *     y = w * o / sqrt(mean(o^2) + eps) * SiLU(z) (pegainfer PR #1003, PR body,
 *     batch_decode/prefill and weights bullets).
 *
 * Everything here is rank-local: head counts are one GPU's share
 * (pegainfer PR #1003, Description: LocalGeometry / RecurrentState /
 * GdrChunkwiseScratch35 sized from rank-local geometry).
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers unless the name ends in _host.
 *   - The caller owns every allocation (pools, activations, scratch, index
 *     arrays).  The library never allocates, frees or synchronises; work is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     runs asynchronously.
 *   - Return 0 (GDN_OK) on success or a negative GDN_E_* code.  Every check
 *     happens before anything is enqueued: on error no kernel runs and no
 *     memory changes (the pages' engines likewise reject a bad head split up
 *     front: pegainfer PR #1003, PR body, config bullet).  gdn_last_error() gives a message for the calling thread.
 *   - Layouts are dense, row-major, innermost index last.  C = 2*Hk*dk +
 *     Hv*dv channels in [q | k | v] order, head-major inside each region.
 *   - "act" arrays use geometry.act_dtype (GDN_F32 or GDN_BF16).
 *   - Rows / sequences with a negative slot are padding: their outputs are
 *     written as zeros and no slot is touched.  A device slot index outside
 *     [0, num_slots) is treated the same way (never dereferenced); pass the
 *     host copy to have it reported as GDN_E_SLOT instead.  Slots not named
 *     by a call are left bit-for-bit unchanged.
 *   - Calls that name the same slot concurrently (on different streams) race.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

enum {
  GDN_OK = 0,
  GDN_E_NULL = -1,        /* a required pointer is NULL */
  GDN_E_SHAPE = -2,       /* a size is out of range (negative count, dim <= 0) */
  GDN_E_HEADS = -3,       /* Hv is not a multiple of Hk */
  GDN_E_UNSUPPORTED = -4, /* dk/dv/K/dtype combination not compiled */
  GDN_E_SLOT = -5,        /* host-visible slot out of range or duplicated */
  GDN_E_OVERLAP = -6,     /* compaction source and destination sets meet */
  GDN_E_SEQLENS = -7,     /* cu_seqlens not 0-based / non-decreasing */
  GDN_E_SCRATCH = -8,     /* scratch or workspace missing or too small */
  GDN_E_HIP = -9,         /* the HIP runtime reported an error at launch */
  GDN_E_ALIGN = -10       /* a device array is not 16-byte aligned (scratch:
                             256-byte) */
};

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Rank-local geometry (pegainfer PR #1003, Description: LocalGeometry with
 * rank-local linear-attention head/dim accessors and indivisibility
 * validation).  Compiled: head_k_dim == head_v_dim in {32, 64, 128};
 * conv_kernel in 2..4; act_dtype GDN_F32 or GDN_BF16. */
typedef struct {
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv; Hv % Hk != 0 -> GDN_E_HEADS */
  int32_t head_k_dim;   /* dk */
  int32_t head_v_dim;   /* dv */
  int32_t conv_kernel;  /* K */
  int32_t act_dtype;    /* gdn_dtype of x, z, a, b, y, conv pool, conv weight */
  float l2norm_eps;     /* q/k l2norm: x / sqrt(sum x^2 + eps) */
  float rmsnorm_eps;    /* gated RMSNorm epsilon */
  float scale;          /* q multiplier; <= 0 means 1/sqrt(dk) */
} gdn_geometry;

/* Per-layer weights, device.  norm_weight is one [dv] vector shared by all
 * V-heads (the norm weight is replicated, not sharded, across ranks:
 * pegainfer PR #1003, PR body, weights bullet). */
typedef struct {
  const void* conv_weight;  /* [C][K] act: depthwise conv1d weight, tap K-1
                               multiplies the current token, no bias */
  const float* A_log;       /* [Hv] f32 */
  const float* dt_bias;     /* [Hv] f32 */
  const float* norm_weight; /* [dv] f32 */
} gdn_layer_weights;

/* Per-layer slot pool, device, caller-owned (pegainfer issue #1001, Splits,
 * "TP CUDA Graph": slot-indexed per-rank recurrent/conv state with
 * scheduler-owned slot_idx). */
typedef struct {
  float* recurrent;   /* [num_slots][Hv][dk][dv] f32: state S, dv innermost */
  void* conv;         /* [num_slots][K][C] act: the last K raw (pre-conv)
                         inputs, oldest first */
  int32_t num_slots;
} gdn_state_pool;

/* ------------------------------------------------------------- sizes */

/* Bytes of one slot in the recurrent pool and in the conv pool, for the
 * caller's capacity math (the pages size worker capacity from these
 * rank-local byte counts: pegainfer PR #1003, PR body, tp_executor bullet). */
int gdn_slot_bytes(const gdn_geometry* geom, size_t* recurrent_bytes,
                   size_t* conv_bytes);

/* Bytes of device scratch gdn_prefill_chunked needs for `total_tokens`
 * packed tokens in `num_seqs` sequences (the GdrChunkwiseScratch35 of
 * pegainfer PR #1003, Description, sized from rank-local geometry). */
int gdn_prefill_scratch_bytes(const gdn_geometry* geom, int32_t total_tokens,
                              int32_t num_seqs, size_t* bytes);

/* ------------------------------------------------------------- decode */

/* One decode token per row: conv update of the fused [q|k|v] input.
 * For row b with slot s = slot_idx[b]:
 *   window = pool.conv[s] (K columns, oldest first) shifted by one with
 *   qkv_in[b] appended; qkv_out[b][c] = SiLU(sum_j conv_weight[c][j] *
 *   window[j][c]); the shifted window is written back to pool.conv[s].
 * qkv_in  [B][C] act;  qkv_out [B][C] f32 (consumed by gdn_decode_batch).
 * slot_idx [B] int32 device; slot_idx_host: optional host copy, validated
 * (range, duplicates) when given.  B == 0 is a no-op.
 * (the decode-time conv of the layer on slot-indexed conv state:
 * pegainfer issue #1001, Splits; pegainfer PR #1003, PR body.) */
int gdn_conv_update(const gdn_geometry* geom, const gdn_layer_weights* w,
                    const gdn_state_pool* pool, const int32_t* slot_idx,
                    const int32_t* slot_idx_host, int32_t B,
                    const void* qkv_in, float* qkv_out, void* stream);

/* One decode token per row, all rows in one launch (pegainfer issue #1001,
 * Splits, "Batched eager TP decode": one batched run over all decode rows).
 * For row b, V-head h, K-head m = h / (Hv/Hk), slot s = slot_idx[b]:
 *   q, k = l2norm of qkv[b]'s K-head m slices (q times scale), v = qkv[b]'s
 *   V-head h slice; g, beta from a[b][h], b[b][h], A_log[h], dt_bias[h];
 *   pool.recurrent[s][h] <- e^g S + beta k (v - e^g S^T k)^T (in place);
 *   o = S_new^T q;  y[b][h] = norm_weight * o / rms(o) * SiLU(z[b][h]).
 * qkv [B][C] f32 (from gdn_conv_update); z [B][Hv][dv] act; a, b [B][Hv] act;
 * y [B][Hv][dv] act; o_raw [B][Hv][dv] f32 or NULL (pre-norm output). */
int gdn_decode_batch(const gdn_geometry* geom, const gdn_layer_weights* w,
                     const gdn_state_pool* pool, const int32_t* slot_idx,
                     const int32_t* slot_idx_host, int32_t B, const float* qkv,
                     const void* z, const void* a, const void* b, void* y,
                     float* o_raw, void* stream);

/* Bytes of the workspace gdn_decode_step needs for up to B rows: a
 * workspace of this size serves every call with B or fewer rows.  It holds
 * one call's arrival counters (B * Hk * (2 dk / 64) words, rounded up to
 * 256 bytes) and scales with the rows, not with the pool. */
int gdn_decode_workspace_bytes(const gdn_geometry* geom, int32_t B, size_t* bytes);

/* Fused decode step: gdn_conv_update followed by gdn_decode_batch for the
 * same rows, in one launch and without the f32 conv-output round trip (the
 * batched decode chain of pegainfer issue #1001, Splits, "Batched eager TP
 * decode", with the conv and the state update of one layer in a single
 * kernel).  Arguments as in those two calls; qkv_in [B][C] act.  Results
 * equal the two-call sequence.
 * workspace: caller-owned device memory of at least
 * gdn_decode_workspace_bytes(geom, B) bytes, 256-byte aligned, ZERO-FILLED
 * before its first use; every call leaves it zero-filled again, so one
 * allocation serves any number of calls, on any pool, one at a time.  Calls
 * that may run at the same time (other streams) need separate workspaces;
 * they may name the same slot numbers in different pools.  One workgroup
 * runs per (row, V-head); the Hv/Hk workgroups that share a K-head's q/k
 * conv window count their reads of it in the workspace, and the last reader
 * writes the shifted window back.  Nothing in the library keeps state
 * between calls. */
int gdn_decode_step(const gdn_geometry* geom, const gdn_layer_weights* w,
                    const gdn_state_pool* pool, const int32_t* slot_idx,
                    const int32_t* slot_idx_host, int32_t B, const void* qkv_in,
                    const void* z, const void* a, const void* b, void* y,
                    float* o_raw, void* workspace, size_t workspace_bytes,
                    void* stream);

/* gdn_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same step as gdn_decode_step, with its workspace taken
 * from a device array the library holds, GDN_NOALLOC_WORKSPACE_BYTES per
 * GPU (one copy on each GPU it runs on, held until the process ends; set up
 * on the first call on a device, with a clear enqueued on `stream`).  A call
 * whose rows need more workspace than that (gdn_decode_workspace_bytes) is
 * rejected with GDN_E_SCRATCH before anything is enqueued; at Hk = 16 and
 * dk = 128 that is past 4096 rows.  Every call on one GPU shares the array,
 * which each call leaves zero-filled: calls that overlap in time on one GPU
 * (other streams, other threads) race and must not be made.  Allocates
 * nothing. */
#define GDN_NOALLOC_WORKSPACE_BYTES ((size_t)1 << 20)
int gdn_decode_step_noalloc(const gdn_geometry* geom, const gdn_layer_weights* w,
                            const gdn_state_pool* pool, const int32_t* slot_idx,
                            const int32_t* slot_idx_host, int32_t B,
                            const void* qkv_in, const void* z, const void* a,
                            const void* b, void* y, float* o_raw, void* stream);

/* ------------------------------------------------------------- prefill */

/* Chunkwise prefill of N packed sequences (pegainfer PR #1003, PR body,
 * batch_decode/prefill bullet: the prefill chain at local head counts;
 * Description: GdrChunkwiseScratch35).  Sequence n owns tokens
 * [cu_seqlens[n], cu_seqlens[n+1]) of qkv_in [T][C] act, z [T][Hv][dv] act,
 * a, b [T][Hv] act, y [T][Hv][dv] act, o_raw [T][Hv][dv] f32 (or NULL; a bf16
 * layer called without it computes the output side, Q S + P V' and the
 * pre-norm output it norms, at bf16 precision; the state path is unchanged).
 * It starts from slot slot_idx[n]'s recurrent state and conv window, or from
 * zeros when has_init is given and has_init[n] == 0, and writes its final
 * state and window back to that slot.  Results equal running the tokens one
 * by one through gdn_conv_update + gdn_decode_batch.
 * cu_seqlens_host [N+1] is required (0-based, non-decreasing; checked) and
 * cu_seqlens_dev must hold the same values.  slot_idx_host is optional (when
 * given: range and duplicates checked).  scratch: device buffer of at least
 * gdn_prefill_scratch_bytes(geom, T, N) bytes, 256-byte aligned; its contents
 * are not preserved. */
int gdn_prefill_chunked(const gdn_geometry* geom, const gdn_layer_weights* w,
                        const gdn_state_pool* pool,
                        const int32_t* cu_seqlens_host,
                        const int32_t* cu_seqlens_dev, const int32_t* slot_idx,
                        const int32_t* slot_idx_host, const uint8_t* has_init,
                        int32_t N, const void* qkv_in, const void* z,
                        const void* a, const void* b, void* y, float* o_raw,
                        void* scratch, size_t scratch_bytes, void* stream);

/* ------------------------------------------------------------- projections */

/* One weight of gdn_linear: weight [N][K] bf16 row-major (a Linear layer's
 * weight), 16-byte aligned; out [M][ldy] bf16, ldy >= N. */
typedef struct {
  const void* weight;
  void* out;
  int32_t N;
  int32_t ldy;
} gdn_linear_out;

/* The projections around the layer core (cortex commit 95dc874,
 * TpQwen3_5GatedDeltaNet bullet: in_proj_qkv, in_proj_z, in_proj_b and
 * in_proj_a split along the V-heads, out_proj along its input dimension, so
 * on one GPU each is a plain product with that GPU's slice of the weight):
 *   outs[i].out[m][n] = sum_k x[m][k] * outs[i].weight[n][k]
 * for m < M, n < outs[i].N, with bf16 x and weights, f32 accumulation and
 * the result rounded once to bf16.  x [M][ldx] bf16 device, 16-byte
 * aligned, ldx >= K, ldx and K multiples of 8.  outs is a HOST array of
 * 1..4 outputs that all read the same x (one launch for the input
 * projections of a token).  No output may overlap x, a weight or another
 * output (GDN_E_OVERLAP).  M == 0 is a no-op. */
int gdn_linear(const void* x, int32_t M, int32_t K, int32_t ldx,
               const gdn_linear_out* outs, int32_t count, void* stream);

/* ------------------------------------------------------------- retire */

/* D2D state compaction on retire (pegainfer issue #1001, Splits, "TP CUDA
 * Graph": D2D compaction on retire).  For every layer l < L and pair i < n:
 * slot dst[i] of pools[l] receives a bit-exact copy of slot src[i]
 * (recurrent state and conv window).  pools is a HOST array of L pools with
 * one geometry.  src_host/dst_host are required and checked: in range, dst
 * entries distinct, and no slot both a source and a destination (so the
 * copies can run in parallel); src_dev/dst_dev hold the same values. */
int gdn_state_compact(const gdn_geometry* geom, const gdn_state_pool* pools,
                      int32_t L, const int32_t* src_host,
                      const int32_t* dst_host, const int32_t* src_dev,
                      const int32_t* dst_dev, int32_t n, void* stream);

/* ------------------------------------------------------------- checks */

/* Device-side check of a device-resident slot index, for callers that hand
 * the library slot_idx without a host copy (graph replay): the pages'
 * engines fail closed on a bad split rather than run with it (pegainfer PR
 * #1003, PR body, config bullet), and this makes the same rule checkable on
 * the device.  Enqueues on `stream` (two kernels, capturable in a graph, no
 * memset) a check of slot_idx [B] against num_slots: every entry negative
 * (a padding row) or in [0, num_slots), and no non-negative slot named by
 * two rows.  result: device int32 [2], written by the check:
 * result[0] = GDN_OK, or GDN_E_SLOT when some row breaks the rule;
 * result[1] = the smallest such row (a slot out of range, or one that an
 * earlier row already names), INT32_MAX when none.  B <= 2^20. */
int gdn_check_slots(const int32_t* slot_idx, int32_t B, int32_t num_slots,
                    int32_t* result, void* stream);

/* ------------------------------------------------------------- status */

const char* gdn_status_str(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* gdn_last_error(void);
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */

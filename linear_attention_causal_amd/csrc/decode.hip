// Batched decode of the Gated DeltaNet layer on gfx950: one token per row.
//
//   conv_update_kernel  slot-indexed conv window shift + depthwise conv + SiLU
//                       over the fused [q|k|v] channels (pegainfer PR #1003,
//                       PR body: the decode-time conv of the layer on
//                       slot-indexed conv state).
//   decode_kernel       per (row, V-head): l2norm of q/k, softplus gates, one
//                       read-modify-write pass over the f32 state tile
//                       S[dk][dv], and the gated RMSNorm epilogue (pegainfer
//                       issue #1001, Splits, "Batched eager TP decode": one
//                       batched launch over all decode rows).
//   decode_head_kernel  both in one launch, per (row, V-head) (the fused
//                       step).
//
// The state update reads S once: with kappa = S^T k and rho = S^T q taken from
// the old state,
//   u  = beta (v - e^g kappa),   S' = e^g S + k u^T,   o = S'^T q = e^g rho + u (k.q)
// so the kernel is one coalesced f32 read and one write of the tile, the
// bandwidth floor of the step.
#include <mutex>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// ------------------------------------------------------------- conv update

struct ConvParams {
  const void* x;        // [B][C] act
  const void* weight;   // [C][K] act
  void* pool;           // [P][K][C] act
  float* out;           // [B][C] f32
  const int32_t* slot_idx;
  int B, C, num_slots;
};

// One thread owns four consecutive channels of one row; K taps per channel.
template <typename Act, int K>
__global__ __launch_bounds__(256) void conv_update_kernel(ConvParams p) {
  using io = act_io<Act>;
  const int row = blockIdx.y;
  const int ch = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (ch >= p.C) return;
  const int slot = p.slot_idx[row];
  float* out = p.out + (size_t)row * p.C + ch;
  if (slot < 0 || slot >= p.num_slots) {
    *reinterpret_cast<f32x4*>(out) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  void* win = static_cast<char*>(p.pool) + (size_t)slot * K * p.C * io::bytes;
  f32x4 col[K];
#pragma unroll
  for (int j = 1; j < K; ++j) col[j - 1] = io::load4(win, (size_t)j * p.C + ch);
  col[K - 1] = io::load4(p.x, (size_t)row * p.C + ch);
  float wt[4][K];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < K; ++j) wt[c][j] = io::load(p.weight, (size_t)(ch + c) * K + j);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    acc.x = fmaf(wt[0][j], col[j].x, acc.x);
    acc.y = fmaf(wt[1][j], col[j].y, acc.y);
    acc.z = fmaf(wt[2][j], col[j].z, acc.z);
    acc.w = fmaf(wt[3][j], col[j].w, acc.w);
  }
  f32x4 r = {silu(acc.x), silu(acc.y), silu(acc.z), silu(acc.w)};
  *reinterpret_cast<f32x4*>(out) = r;
  // the window stores raw inputs, so re-storing them is lossless
#pragma unroll
  for (int j = 0; j < K; ++j) io::store4(win, (size_t)j * p.C + ch, col[j]);
}

// ------------------------------------------------------------- state step

struct DecodeParams {
  const float* qkv;     // [B][C] f32
  const void* z;        // [B][Hv][dv] act
  const void* a;        // [B][Hv] act
  const void* b;        // [B][Hv] act
  void* y;              // [B][Hv][dv] act
  float* o_raw;         // [B][Hv][dv] f32 or null
  float* rec;           // [P][Hv][D][D] f32
  const int32_t* slot_idx;
  const float* A_log;
  const float* dt_bias;
  const float* norm_w;
  int B, Hk, Hv, C, num_slots, r;
  float l2eps, rmseps, scale;
};

// One workgroup per (row, V-head).  Thread t owns the four state columns
// 4*(t % CG) .. +3 of rows (t / CG) + RG*i: each wave instruction moves whole
// contiguous rows, and the whole tile is requested before any arithmetic.
template <typename Act, int D, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeParams p) {
  using io = act_io<Act>;
  constexpr int CG = D / 4;         // column groups of four floats
  constexpr int RG = NT / CG;       // row groups
  constexpr int RPT = D / RG;       // rows per thread
  constexpr int NW = NT / 64;       // waves
  constexpr int QKV_PER = (3 * D + NT - 1) / NT;
  static_assert(NT % CG == 0 && D % RG == 0 && CG <= 64 && NT % 64 == 0, "layout");

  __shared__ float s_qkv[3 * D];
  __shared__ f32x4 s_red[NW][2][CG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;
  const int row = blockIdx.x / p.Hv;
  const int h = blockIdx.x - row * p.Hv;
  const size_t out_off = ((size_t)row * p.Hv + h) * D;
  const int slot = p.slot_idx[row];
  if (slot < 0 || slot >= p.num_slots) {  // padding row: zeros, no state access
    for (int j = tid; j < D; j += NT) {
      io::store(p.y, out_off + j, 0.f);
      if (p.o_raw) p.o_raw[out_off + j] = 0.f;
    }
    return;
  }
  const int m = h / p.r;  // K-head read by V-head h (repeat_interleave)

  // q, k (K-head m) and v (V-head h) and the gate inputs: issued before the
  // state tile, unconditionally (indices past 3D are clamped and their
  // values dropped; a load under a branch would be waited for at once)
  const float* xr = p.qkv + (size_t)row * p.C;
  float tmp[QKV_PER];
#pragma unroll
  for (int e = 0; e < QKV_PER; ++e) {
    const int j = min(tid + e * NT, 3 * D - 1);
    const int part = j / D, jj = j - part * D;
    const size_t off = part == 0 ? (size_t)m * D + jj
                     : part == 1 ? (size_t)(p.Hk + m) * D + jj
                                 : (size_t)2 * p.Hk * D + (size_t)h * D + jj;
    tmp[e] = xr[off];
  }
  const float A_log = p.A_log[h], dt_bias = p.dt_bias[h];
  const float a_in = io::load(p.a, (size_t)row * p.Hv + h);
  const float b_in = io::load(p.b, (size_t)row * p.Hv + h);
  float* S = p.rec + ((size_t)slot * p.Hv + h) * D * D;
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)  // streamed once: nontemporal
    s[i] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(S + (size_t)(rg + RG * i) * D + 4 * cg));

  float g, beta;
  gates(A_log, dt_bias, a_in, b_in, g, beta);
  const float eg = expf(g);

#pragma unroll
  for (int e = 0; e < QKV_PER; ++e) {
    const int j = tid + e * NT;
    if (j < 3 * D) s_qkv[j] = tmp[e];
  }
  __syncthreads();

  // l2 norms and k.q, every wave on its own (no second barrier)
  float sqq = 0.f, skk = 0.f, sqk = 0.f;
  for (int j = lane; j < D; j += 64) {
    const float qv = s_qkv[j], kv = s_qkv[D + j];
    sqq = fmaf(qv, qv, sqq);
    skk = fmaf(kv, kv, skk);
    sqk = fmaf(qv, kv, sqk);
  }
  sqq = wave_sum(sqq);
  skk = wave_sum(skk);
  sqk = wave_sum(sqk);
  const float rq = p.scale / sqrtf(sqq + p.l2eps);
  const float rk = 1.0f / sqrtf(skk + p.l2eps);
  const float kq = sqk * rq * rk;  // k_hat . q_hat

  // kappa = S^T k_hat, rho = S^T q_hat over this thread's rows
  f32x4 kap = {0.f, 0.f, 0.f, 0.f}, rho = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r_ = rg + RG * i;
    const float kk = s_qkv[D + r_] * rk, qq = s_qkv[r_] * rq;
    kap += s[i] * kk;
    rho += s[i] * qq;
  }
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
    kap.x += __shfl_xor(kap.x, off, 64); kap.y += __shfl_xor(kap.y, off, 64);
    kap.z += __shfl_xor(kap.z, off, 64); kap.w += __shfl_xor(kap.w, off, 64);
    rho.x += __shfl_xor(rho.x, off, 64); rho.y += __shfl_xor(rho.y, off, 64);
    rho.z += __shfl_xor(rho.z, off, 64); rho.w += __shfl_xor(rho.w, off, 64);
  }
  if (lane < CG) {
    s_red[wave][0][cg] = kap;
    s_red[wave][1][cg] = rho;
  }
  __syncthreads();
  kap = s_red[0][0][cg];
  rho = s_red[0][1][cg];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    kap += s_red[w][0][cg];
    rho += s_red[w][1][cg];
  }

  const f32x4 v = *reinterpret_cast<const f32x4*>(&s_qkv[2 * D + 4 * cg]);
  const f32x4 u = beta * (v - eg * kap);
  const f32x4 o = eg * rho + u * kq;

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r_ = rg + RG * i;
    const float kk = s_qkv[D + r_] * rk;
    f32x4 ns;
    ns.x = fmaf(eg, s[i].x, kk * u.x);
    ns.y = fmaf(eg, s[i].y, kk * u.y);
    ns.z = fmaf(eg, s[i].z, kk * u.z);
    ns.w = fmaf(eg, s[i].w, kk * u.w);
    __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + (size_t)r_ * D + 4 * cg));
  }

  // gated RMSNorm over the D outputs of this head (wave 0; every row group
  // of the wave holds all columns, so the xor-reduction over the CG lanes of
  // a group yields the full sum)
  if (wave == 0) {
    float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
    for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.0f / sqrtf(ss / D + p.rmseps);
    if (lane < CG) {
      const f32x4 nw = *reinterpret_cast<const f32x4*>(p.norm_w + 4 * cg);
      const f32x4 zz = io::load4(p.z, out_off + 4 * cg);
      f32x4 yv;
      yv.x = nw.x * o.x * inv * silu(zz.x);
      yv.y = nw.y * o.y * inv * silu(zz.y);
      yv.z = nw.z * o.z * inv * silu(zz.z);
      yv.w = nw.w * o.w * inv * silu(zz.w);
      io::store4(p.y, out_off + 4 * cg, yv);
      if (p.o_raw) *reinterpret_cast<f32x4*>(p.o_raw + out_off + 4 * cg) = o;
    }
  }
}

// ------------------------------------------------------------- fused step

// Nontemporal element and four-element stores of an activation: the fused
// step's small writes (conv windows, y) leave no dirty lines in L2 for the
// end of the kernel to write back, as its tile stores already do (measured
// 7.98 -> 7.83 us at 16 rows).
template <typename Act> __device__ __forceinline__ void store_nt(void* p, size_t i, float v);
template <> __device__ __forceinline__ void store_nt<float>(void* p, size_t i, float v) {
  __builtin_nontemporal_store(v, static_cast<float*>(p) + i);
}
template <> __device__ __forceinline__ void store_nt<__bf16>(void* p, size_t i, float v) {
  __builtin_nontemporal_store(static_cast<unsigned short>(f32_to_bf16_bits(v)),
                              static_cast<unsigned short*>(p) + i);
}
template <typename Act> __device__ __forceinline__ void store4_nt(void* p, size_t i, f32x4 v);
template <> __device__ __forceinline__ void store4_nt<float>(void* p, size_t i, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(p) + i));
}
// i is a multiple of 4: two aligned 32-bit words of packed bf16 pairs
template <> __device__ __forceinline__ void store4_nt<__bf16>(void* p, size_t i, f32x4 v) {
  unsigned int* w = reinterpret_cast<unsigned int*>(static_cast<unsigned short*>(p) + i);
  __builtin_nontemporal_store(f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16), w);
  __builtin_nontemporal_store(f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16), w + 1);
}

struct StepParams {
  const void* x;        // [B][C] act (fused [q|k|v] input of this token)
  const void* weight;   // [C][K] act
  void* conv;           // [P][K][C] act
  const void* z;        // [B][Hv][dv] act
  const void* a;        // [B][Hv] act
  const void* b;        // [B][Hv] act
  void* y;              // [B][Hv][dv] act
  float* o_raw;         // [B][Hv][dv] f32 or null
  float* rec;           // [P][Hv][D][D] f32
  const int32_t* slot_idx;
  const float* A_log;
  const float* dt_bias;
  const float* norm_w;
  unsigned int* arrivals;   // workspace [B][Hk][2D/64]: readers of a q/k window
  int B, Hk, Hv, C, num_slots;
  int r;                // Hv / Hk
  int per_xcd;          // (row, V-head) units per XCD lane of the grid
  float l2eps, rmseps, scale;
};

// One workgroup of 2D threads per (row, V-head): the whole state tile of one
// head is read once and written once by the same workgroup, which also
// holds every output of the head for the gated RMSNorm.
//
// q/k conv window.  The r = Hv/Hk workgroups of one (row, K-head) each
// convolve the K-head's q/k channels from the old window, and the shifted
// window may be written back only after all r have read it.  Each wave
// holds 64 q/k channels and, once its loads of them have returned, adds one
// to the counter of (row, K-head, wave) in the caller's workspace; the
// arrival that finds r-1 (mod r) earlier arrivals is the last reader,
// writes those channels' shifted window and takes r back off the counter,
// so the counters are zero between calls and nobody waits for anybody.  A
// v channel has one reader, its V-head's workgroup, which writes it back
// itself.  Block x runs unit (x % 8) * per_xcd + x / 8, which keeps the r
// units of a (row, K-head) on one XCD (blocks are dealt to the eight XCDs
// in turn) and so their window reads in one L2.
template <typename Act, int D, int K>
__global__ __launch_bounds__(2 * D) void decode_head_kernel(StepParams p) {
  using io = act_io<Act>;
  constexpr int NT = 2 * D;          // threads
  constexpr int CGH = D / 4;         // four-column groups
  constexpr int RG = NT / CGH;       // row groups
  constexpr int RPT = D / RG;        // rows per thread
  constexpr int HW = NT / 64;        // waves (each holds 64 of the 2D q/k channels)
  static_assert(NT % 64 == 0 && CGH <= 64 && 64 % CGH == 0 && RPT >= 1, "layout");

  __shared__ float s_x[3 * D];       // conv + SiLU output: q, k, v_h
  __shared__ f32x4 s_red[HW][2][CGH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cgh = tid % CGH, rg = tid / CGH;
  const int unit = (blockIdx.x & 7) * p.per_xcd + (blockIdx.x >> 3);
  if (unit >= p.B * p.Hv) return;
  const int row = unit / p.Hv;
  const int h = unit - row * p.Hv;
  const int m = h / p.r;
  const size_t out_off = ((size_t)row * p.Hv + h) * D;
  const int slot = p.slot_idx[row];
  if (slot < 0 || slot >= p.num_slots) {  // padding row: zeros, no state access
    if (tid < D) {
      io::store(p.y, out_off + tid, 0.f);
      if (p.o_raw) p.o_raw[out_off + tid] = 0.f;
    }
    return;
  }

  // 1. conv inputs (window columns 1..K-1, the token, the weights), then the
  // tile.  Thread t holds q/k channel t of [q_m | k_m] and, for t < D, v
  // channel t of V-head h (loads from a clamped channel, so unconditional).
  // The small inputs stay unconverted until the tile's loads are out (a
  // conversion scheduled among those loads would wait for its own).
  void* win = static_cast<char*>(p.conv) + (size_t)slot * K * p.C * io::bytes;
  const int chq = tid < D ? m * D + tid : (p.Hk + m) * D + tid - D;
  const int chv = 2 * p.Hk * D + h * D + (tid < D ? tid : D - 1);
  typename io::raw_t rcq[K], rwq[K], rcv[K], rwv[K];
#pragma unroll
  for (int k = 1; k < K; ++k) {
    rcq[k - 1] = io::load_raw(win, (size_t)k * p.C + chq);
    rcv[k - 1] = io::load_raw(win, (size_t)k * p.C + chv);
  }
  rcq[K - 1] = io::load_raw(p.x, (size_t)row * p.C + chq);
  rcv[K - 1] = io::load_raw(p.x, (size_t)row * p.C + chv);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    rwq[k] = io::load_raw(p.weight, (size_t)chq * K + k);
    rwv[k] = io::load_raw(p.weight, (size_t)chv * K + k);
  }
  const typename io::raw_t ra = io::load_raw(p.a, (size_t)row * p.Hv + h);
  const typename io::raw_t rb = io::load_raw(p.b, (size_t)row * p.Hv + h);
  const float A_log = p.A_log[h], dt_bias = p.dt_bias[h];
  // the epilogue's z and norm weight too (every thread, its four columns),
  // so the end of the kernel waits on no load
  const typename io::raw4_t rz = io::load4_raw(p.z, out_off + 4 * cgh);
  const f32x4 nw = *reinterpret_cast<const f32x4*>(p.norm_w + 4 * cgh);
  __builtin_amdgcn_sched_barrier(0);
  float* S = p.rec + ((size_t)slot * p.Hv + h) * D * D;
  // issued in the order the reduction consumes them (the scheduler otherwise
  // reverses it and the first product waits for the whole tile); nothing
  // moves across the barriers
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    s[i] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(S + (size_t)(rg + RG * i) * D + 4 * cgh));
    __builtin_amdgcn_sched_barrier(0);
  }
  float cq[K], wq[K], cv[K], wv[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    cq[k] = io::from_raw(rcq[k]);
    cv[k] = io::from_raw(rcv[k]);
    wq[k] = io::from_raw(rwq[k]);
    wv[k] = io::from_raw(rwv[k]);
  }
  const float a_in = io::from_raw(ra), b_in = io::from_raw(rb);
  const f32x4 zz = io::from_raw4(rz);

  // 2. conv + SiLU
  float accq = 0.f, accv = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    accq = fmaf(wq[k], cq[k], accq);
    accv = fmaf(wv[k], cv[k], accv);
  }
  s_x[tid] = silu(accq);
  if (tid < D) s_x[2 * D + tid] = silu(accv);
  // the shifted v window, by the thread that owns each channel, as soon as its
  // own loads of it have returned (accv used them).  Threads past D loaded
  // channel D-1 only as a clamp and never use it, so they store nothing.
  // Stored this early, these writes are not queued behind the tile's.
  if (tid < D) {
#pragma unroll
    for (int k = 0; k < K; ++k) store_nt<Act>(win, (size_t)k * p.C + chv, cv[k]);
  }
  // arrival (lane 0 of each wave; one atomic per wave); the increment takes
  // accq as an operand (through an empty asm), so it issues only after this
  // wave's q/k window loads have returned
  unsigned int* ctr = p.arrivals + ((size_t)row * p.Hk + m) * HW + wave;
  unsigned int arrived = 0;
  unsigned int one = 1;
  asm volatile("" : "+v"(one) : "v"(accq));
  if (lane == 0 && p.r > 1)
    arrived = __hip_atomic_fetch_add(ctr, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float g, beta;
  gates(A_log, dt_bias, a_in, b_in, g, beta);
  const float eg = expf(g);
  __syncthreads();

  const float* sq = s_x;
  const float* sk = s_x + D;
  const float* sv = s_x + 2 * D;
  float sqq = 0.f, skk = 0.f, sqk = 0.f;
  for (int j = lane; j < D; j += 64) {
    const float qv = sq[j], kv = sk[j];
    sqq = fmaf(qv, qv, sqq);
    skk = fmaf(kv, kv, skk);
    sqk = fmaf(qv, kv, sqk);
  }
  sqq = wave_sum(sqq);
  skk = wave_sum(skk);
  sqk = wave_sum(sqk);
  const float rq = p.scale / sqrtf(sqq + p.l2eps);
  const float rk = 1.0f / sqrtf(skk + p.l2eps);
  const float kq = sqk * rq * rk;
  float kr[RPT], qr[RPT];   // k_hat, q_hat at this thread's rows
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    kr[i] = sk[rg + RG * i] * rk;
    qr[i] = sq[rg + RG * i] * rq;
  }

  // 3. reduce (kappa = S^T k, rho = S^T q)
  f32x4 kap = {0.f, 0.f, 0.f, 0.f}, rho = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    kap += s[i] * kr[i];
    rho += s[i] * qr[i];
  }
#pragma unroll
  for (int off = CGH; off < 64; off <<= 1) {
    kap.x += __shfl_xor(kap.x, off, 64); kap.y += __shfl_xor(kap.y, off, 64);
    kap.z += __shfl_xor(kap.z, off, 64); kap.w += __shfl_xor(kap.w, off, 64);
    rho.x += __shfl_xor(rho.x, off, 64); rho.y += __shfl_xor(rho.y, off, 64);
    rho.z += __shfl_xor(rho.z, off, 64); rho.w += __shfl_xor(rho.w, off, 64);
  }
  if (lane < CGH) {
    s_red[wave][0][cgh] = kap;
    s_red[wave][1][cgh] = rho;
  }
  __syncthreads();
  kap = s_red[0][0][cgh];
  rho = s_red[0][1][cgh];
#pragma unroll
  for (int w = 1; w < HW; ++w) {
    kap += s_red[w][0][cgh];
    rho += s_red[w][1][cgh];
  }
  const f32x4 v = *reinterpret_cast<const f32x4*>(&sv[4 * cgh]);
  const f32x4 u = beta * (v - eg * kap);
  const f32x4 o = eg * rho + u * kq;

  // The small writes go out before the tile's 16 stores per thread, so the
  // kernel's end does not wait for them behind those (measured: 0.4 us of the
  // 8.4 us step at 16 rows when they came last).
  // 4. the last reader of this wave's q/k channels writes their shifted
  // window.  Its arrival's return follows the tile loads consumed above, so
  // waiting for it here costs nothing.
  bool last = true;
  if (p.r > 1) {
    const unsigned int before = __builtin_amdgcn_readfirstlane(arrived);
    last = before % (unsigned int)p.r == (unsigned int)(p.r - 1);
  }
  if (last) {
#pragma unroll
    for (int k = 0; k < K; ++k) store_nt<Act>(win, (size_t)k * p.C + chq, cq[k]);
    if (p.r > 1 && lane == 0)
      __hip_atomic_fetch_add(ctr, 0u - (unsigned int)p.r, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }

  // 5. gated RMSNorm over the D outputs (first wave, before its tile stores;
  // each row group holds all columns, so the xor-reduction over its CGH lanes
  // gives the full sum)
  if (wave == 0) {
    float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
    for (int off = 1; off < CGH; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.0f / sqrtf(ss / D + p.rmseps);
    if (lane < CGH) {
      f32x4 yv;
      yv.x = nw.x * o.x * inv * silu(zz.x);
      yv.y = nw.y * o.y * inv * silu(zz.y);
      yv.z = nw.z * o.z * inv * silu(zz.z);
      yv.w = nw.w * o.w * inv * silu(zz.w);
      store4_nt<Act>(p.y, out_off + 4 * cgh, yv);
      if (p.o_raw) *reinterpret_cast<f32x4*>(p.o_raw + out_off + 4 * cgh) = o;
    }
  }

  // 6. the new tile
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    f32x4 ns;
    ns.x = fmaf(eg, s[i].x, kr[i] * u.x);
    ns.y = fmaf(eg, s[i].y, kr[i] * u.y);
    ns.z = fmaf(eg, s[i].z, kr[i] * u.z);
    ns.w = fmaf(eg, s[i].w, kr[i] * u.w);
    __builtin_nontemporal_store(
        ns, reinterpret_cast<f32x4*>(S + (size_t)(rg + RG * i) * D + 4 * cgh));
  }
}

// Workspace of gdn_decode_step: the arrival counters [B][Hk][2D/64] u32
// (row-keyed, so its size follows the rows of a call and a workspace for B
// rows serves every smaller call).
size_t decode_workspace_bytes(const gdn_geometry& g, long long B) {
  const long long words = B * g.num_k_heads * (2LL * g.head_k_dim / 64);
  return ((size_t)words * 4 + 255) & ~size_t(255);
}

template <typename Act, int D>
static hipError_t head_k(const StepParams& p, int K, hipStream_t st) {
  dim3 grid(8 * p.per_xcd);
  switch (K) {
    case 2: decode_head_kernel<Act, D, 2><<<grid, 2 * D, 0, st>>>(p); break;
    case 3: decode_head_kernel<Act, D, 3><<<grid, 2 * D, 0, st>>>(p); break;
    case 4: decode_head_kernel<Act, D, 4><<<grid, 2 * D, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename Act>
static hipError_t head_d(const StepParams& p, int D, int K, hipStream_t st) {
  switch (D) {
    case 32: return head_k<Act, 32>(p, K, st);
    case 64: return head_k<Act, 64>(p, K, st);
    case 128: return head_k<Act, 128>(p, K, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_step(const gdn_geometry& g, const gdn_layer_weights& w,
                              const gdn_state_pool& pool, const int32_t* slot_idx, int B,
                              const void* qkv_in, const void* z, const void* a, const void* b,
                              void* y, float* o_raw, void* workspace, hipStream_t stream) {
  StepParams p;
  p.x = qkv_in;
  p.weight = w.conv_weight;
  p.conv = pool.conv;
  p.z = z;
  p.a = a;
  p.b = b;
  p.y = y;
  p.o_raw = o_raw;
  p.rec = pool.recurrent;
  p.slot_idx = slot_idx;
  p.A_log = w.A_log;
  p.dt_bias = w.dt_bias;
  p.norm_w = w.norm_weight;
  p.arrivals = static_cast<unsigned int*>(workspace);
  p.B = B;
  p.Hk = g.num_k_heads;
  p.Hv = g.num_v_heads;
  p.C = 2 * g.num_k_heads * g.head_k_dim + g.num_v_heads * g.head_v_dim;
  p.num_slots = pool.num_slots;
  p.l2eps = g.l2norm_eps;
  p.rmseps = g.rmsnorm_eps;
  p.scale = g.scale > 0.f ? g.scale : 1.0f / sqrtf((float)g.head_k_dim);
  p.r = g.num_v_heads / g.num_k_heads;
  const long long units = (long long)B * p.Hv;
  const long long per = (units + 7) / 8;
  p.per_xcd = (int)((per + p.r - 1) / p.r * p.r);   // a (row, K-head) never straddles two XCDs
  if (g.act_dtype == GDN_BF16) return head_d<__bf16>(p, g.head_k_dim, g.conv_kernel, stream);
  return head_d<float>(p, g.head_k_dim, g.conv_kernel, stream);
}

// ------------------------------------------------------------- no-alloc step

// Workspace of gdn_decode_step_noalloc: one array per GPU in the code object,
// held until the process ends.  Host code never names it as an address (the
// name is a host-side stand-in); it uses the per-device pointer that
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4* p, size_t n) {
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device
}  // namespace

// The calling thread's current device's copy of the array, set up on the
// first call for that device: its address taken once with the device
// current, and the array cleared once (a fill kernel on `stream`, ahead of
// the step; no memset node, so the clear may also be captured).
hipError_t static_scratch(void** ptr, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    fill_zero_kernel<<<64, 256, 0, stream>>>(static_cast<u32x4*>(p), kStaticScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ------------------------------------------------------------- launchers

template <typename Act>
static hipError_t conv_dispatch(const ConvParams& p, int K, hipStream_t st) {
  dim3 grid((p.C / 4 + 255) / 256, p.B);
  switch (K) {
    case 2: conv_update_kernel<Act, 2><<<grid, 256, 0, st>>>(p); break;
    case 3: conv_update_kernel<Act, 3><<<grid, 256, 0, st>>>(p); break;
    case 4: conv_update_kernel<Act, 4><<<grid, 256, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_conv_update(const gdn_geometry& g, const gdn_layer_weights& w,
                              const gdn_state_pool& pool, const int32_t* slot_idx,
                              int B, const void* qkv_in, float* qkv_out,
                              hipStream_t stream) {
  ConvParams p;
  p.x = qkv_in;
  p.weight = w.conv_weight;
  p.pool = pool.conv;
  p.out = qkv_out;
  p.slot_idx = slot_idx;
  p.B = B;
  p.C = 2 * g.num_k_heads * g.head_k_dim + g.num_v_heads * g.head_v_dim;
  p.num_slots = pool.num_slots;
  if (g.act_dtype == GDN_BF16) return conv_dispatch<__bf16>(p, g.conv_kernel, stream);
  return conv_dispatch<float>(p, g.conv_kernel, stream);
}

template <typename Act>
static hipError_t decode_dispatch(const DecodeParams& p, int D, hipStream_t st) {
  dim3 grid(p.B * p.Hv);
  switch (D) {
    case 32: decode_kernel<Act, 32, 64><<<grid, 64, 0, st>>>(p); break;
    case 64: decode_kernel<Act, 64, 128><<<grid, 128, 0, st>>>(p); break;
    case 128: decode_kernel<Act, 128, 256><<<grid, 256, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const gdn_geometry& g, const gdn_layer_weights& w,
                         const gdn_state_pool& pool, const int32_t* slot_idx, int B,
                         const float* qkv, const void* z, const void* a,
                         const void* b, void* y, float* o_raw, hipStream_t stream) {
  DecodeParams p;
  p.qkv = qkv;
  p.z = z;
  p.a = a;
  p.b = b;
  p.y = y;
  p.o_raw = o_raw;
  p.rec = pool.recurrent;
  p.slot_idx = slot_idx;
  p.A_log = w.A_log;
  p.dt_bias = w.dt_bias;
  p.norm_w = w.norm_weight;
  p.B = B;
  p.Hk = g.num_k_heads;
  p.Hv = g.num_v_heads;
  p.C = 2 * g.num_k_heads * g.head_k_dim + g.num_v_heads * g.head_v_dim;
  p.num_slots = pool.num_slots;
  p.r = g.num_v_heads / g.num_k_heads;
  p.l2eps = g.l2norm_eps;
  p.rmseps = g.rmsnorm_eps;
  p.scale = g.scale > 0.f ? g.scale : 1.0f / sqrtf((float)g.head_k_dim);
  if (g.act_dtype == GDN_BF16) return decode_dispatch<__bf16>(p, g.head_k_dim, stream);
  return decode_dispatch<float>(p, g.head_k_dim, stream);
}

}  // namespace gdn

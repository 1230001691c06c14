// Chunkwise prefill of the Gated DeltaNet layer on gfx950 (the GDR prefill
// chain with its chunkwise scratch: pegainfer PR #1003, PR body,
// batch_decode/prefill bullet, and Description, GdrChunkwiseScratch35).
//
// Blocked form of the gated delta rule over chunks of L = 64 tokens that
// never span two sequences (the WY representation of the chunk, Gated
// DeltaNet paper, chunkwise training section).  Inside a chunk, with gamma_i
// the running sum of the gates g and beta_i the write strengths (both per
// V-head),
//   A   = strict_lower(beta_i e^{gamma_i - gamma_j} k_i . k_j)
//   Tm  = (I + A)^{-1}                                  (unit lower triangular)
//   W   = Tm diag(beta e^gamma) K,   U = Tm diag(beta) V
//   V'  = U - W S                                        (the writes u_t)
//   O   = diag(e^gamma) Q S + P V',   P = mask_{j<=i}(e^{gamma_i-gamma_j}) * (Q K^T)
//   S  <- e^{gamma_last} S + K^T diag(e^{gamma_last-gamma}) V'
// which is the token recurrence S_t = e^{g_t}S_{t-1} + beta_t k_t (v_t -
// e^{g_t} S_{t-1}^T k_t)^T, o_t = S_t^T q_t unrolled over the chunk.  Decays
// are only formed as e^{gamma_i - gamma_j} with j <= i (<= 1).
//
// Launches, in stream order:
//   0. plan   one workgroup: chunk_base[n] = number of chunks before sequence n
//             (only for batches of more than kInlineSeqs sequences; smaller
//             ones carry the prefix, taken from the host copy, in the launch).
//   1. q/k    (chunk, K-head), all chunks in parallel: conv + SiLU of q/k, l2
//             norms, q_hat and k_hat^T fragments, K K^T and Q K^T.
//   1'. WY    (chunk, V-head), all chunks in parallel: the gates and
//             their running sum, A, P, Tm (blocked 16 x 16 triangular
//             inverse), conv + SiLU of v, W and U.  Operands are written as
//             bf16 (hi, lo) pairs (U as f32) in the fragment layout of the
//             next kernel.
//   2. state  (sequence, V-head, 16 NCB dv columns), sequential over the
//             chunks of a sequence, the dv columns of S split over
//             workgroups (they evolve independently): V' = U - W S and the
//             state carry on one half of the waves, O = e^gamma Q S + P V' on
//             the other half, on 3-pass bf16 MFMA (x = hi + lo; hi*hi + hi*lo
//             + lo*hi with f32 accumulation, about 2^-16 relative), O
//             (pre-norm) to the caller's f32 o_raw, or to a bf16 copy in the
//             scratch when a bf16 layer is called without one.
//   3. norm   (chunk, V-head): gated RMSNorm with SiLU(z) -> y.
// The per-chunk launches (1, 1', 3) cover the real chunks of the batch when
// the prefix travels with the launch, else every (chunk slot, sequence) pair
// up to the longest sequence (see chunk_of).
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kL = 64;        // chunk length
constexpr int kNT = 256;      // threads per workgroup of the q/k, WY and norm kernels
constexpr int kNW = kNT / 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Chunk-indexed scratch: chunk g = chunk_base[n] + c holds 64 rows (rows past
// the end of a sequence are written as zeros by the q/k and WY kernels).  Everything
// the sequential state kernel reads is stored fragment-major (see frag_at):
// one wave's MFMA operand tile is one contiguous 1 KB block.
struct PrefillScratch {
  int32_t* chunk_base;     // [N+1]
  __bf16* qh[2];           // hi, lo: [G][Hk] 64 x D    q_hat, A-operand blocks
  __bf16* kt[2];           //         [G][Hk] D x 64    k_hat^T, A-operand blocks
  __bf16* w[2];            //         [G][Hv] 64 x D    -Tm diag(beta e^gamma) K
  __bf16* pm[2];           //         [G][Hv] 64 x 64   masked, decayed Q K^T
  float* ut;               // [G][Hv] 64 x D Tm diag(beta) V, accumulator blocks
  float* gq;               // [G][Hk][2][64][64] K K^T and Q K^T (lower blocks), f32
  float* gam;              // [G][Hv][64] running sum of g
  float* o;                // [T][Hv][D] pre-norm output
};

static size_t chunk_bound(long long T, long long N) { return (size_t)((T + kL - 1) / kL + N); }

constexpr int kScratchParts = 13;

struct ScratchPlan {
  size_t off[kScratchParts];
  size_t total;
};

static ScratchPlan plan_scratch(const gdn_geometry& g, long long T, long long N) {
  const size_t G = chunk_bound(T, N), D = (size_t)g.head_k_dim;
  const size_t Hk = (size_t)g.num_k_heads, Hv = (size_t)g.num_v_heads;
  const size_t sizes[kScratchParts] = {
      (size_t)(N + 1) * 4,
      G * Hk * kL * D * 2, G * Hk * kL * D * 2,      // qh
      G * Hk * D * kL * 2, G * Hk * D * kL * 2,      // kt
      G * Hv * kL * D * 2, G * Hv * kL * D * 2,      // w
      G * Hv * kL * kL * 2, G * Hv * kL * kL * 2,    // pm
      G * Hv * D * kL * 4,                           // ut
      G * Hk * 2 * kL * kL * 4,                      // gq
      G * Hv * kL * 4,                               // gam
      (size_t)T * Hv * D * 4};                       // o
  ScratchPlan sp;
  size_t at = 0;
  for (int i = 0; i < kScratchParts; ++i) {
    sp.off[i] = at;
    at += align256(sizes[i]);
  }
  sp.total = at;
  return sp;
}

size_t prefill_scratch_bytes(const gdn_geometry& g, long long T, long long N) {
  return plan_scratch(g, T, N).total;
}

static PrefillScratch carve(const gdn_geometry& g, long long T, long long N, void* base) {
  const ScratchPlan sp = plan_scratch(g, T, N);
  char* c = static_cast<char*>(base);
  PrefillScratch s;
  s.chunk_base = reinterpret_cast<int32_t*>(c + sp.off[0]);
  for (int k = 0; k < 2; ++k) {
    s.qh[k] = reinterpret_cast<__bf16*>(c + sp.off[1 + k]);
    s.kt[k] = reinterpret_cast<__bf16*>(c + sp.off[3 + k]);
    s.w[k] = reinterpret_cast<__bf16*>(c + sp.off[5 + k]);
    s.pm[k] = reinterpret_cast<__bf16*>(c + sp.off[7 + k]);
  }
  s.ut = reinterpret_cast<float*>(c + sp.off[9]);
  s.gq = reinterpret_cast<float*>(c + sp.off[10]);
  s.gam = reinterpret_cast<float*>(c + sp.off[11]);
  s.o = reinterpret_cast<float*>(c + sp.off[12]);
  return s;
}

constexpr int kInlineSeqs = 64;

struct PrefillParams {
  const void* x;        // [T][C] act
  const void* z;        // [T][Hv][D] act
  const void* a;        // [T][Hv] act
  const void* b;        // [T][Hv] act
  void* y;              // [T][Hv][D] act
  float* obuf;          // [T][Hv][D] f32: caller's o_raw or scratch
  // bf16 layers called without o_raw: the output-only products (Q S and
  // P V') run single-pass on the hi halves and the pre-norm output is kept
  // as bf16 in the scratch; it feeds only the gated RMSNorm, whose bf16
  // result it perturbs by a few 2^-9 relative.  The state path (W S, the
  // state update, and everything that feeds them) stays 3-pass.
  bool o_bf16;
  float* rec;           // [P][Hv][D][D]
  void* conv;           // [P][K][C] act
  const int32_t* cu;    // [N+1]
  const int32_t* slot_idx;
  const uint8_t* has_init;
  const void* conv_w;   // [C][K] act
  const float* A_log;
  const float* dt_bias;
  const float* norm_w;
  PrefillScratch s;
  long long T;
  size_t G;             // chunk capacity of the scratch
  // Small batches: sequence bounds and chunk prefix from the validated host
  // copy of cu_seqlens, passed with the launch (no plan kernel, no device
  // read of cu_seqlens); larger ones use the device copy and the plan kernel.
  bool inl;
  int32_t inl_cu[kInlineSeqs + 1];
  int32_t inl_cb[kInlineSeqs + 1];
  // the state pass's sequence order, longest first: its workgroups are
  // dispatched in this order, so the longest chain of chunks starts first
  int32_t inl_order[kInlineSeqs];
  int N, Hk, Hv, C, num_slots, r;
  int max_chunks;       // chunks of the longest sequence
  float l2eps, rmseps, scale;
};

struct SeqInfo {
  long long begin;  // first packed token
  int len;
  int slot;         // < 0: padding (no state)
  bool init;
};

// Device copy of an index array read in the branch beside an inline one: the
// volatile read keeps the compiler from merging the two branches into one
// load through a select of the two addresses (a generic pointer whose load
// waits a vector-memory round trip; the inline read alone is a scalar load).
__device__ __forceinline__ long long read_dev(const int32_t* a, int i) {
  return *reinterpret_cast<const volatile int32_t*>(a + i);
}

// First scratch chunk of sequence n.
__device__ __forceinline__ size_t chunk_base_of(const PrefillParams& p, int n) {
  if (p.inl) return (size_t)p.inl_cb[n];
  return (size_t)read_dev(p.s.chunk_base, n);
}

// (sequence n, chunk c) of this workgroup for the per-chunk kernels.  A
// launch that carries the chunk prefix enumerates only real chunks along x
// (packed varlen batches would otherwise launch max_chunks per sequence,
// mostly empty workgroups that still read their sequence's bounds); n is
// the last sequence whose first chunk is at or before x.  Otherwise x is
// the chunk and y the sequence.
__device__ __forceinline__ void chunk_at(const PrefillParams& p, int g, int& n, int& c) {
  int lo = 0, hi = p.N;   // inl_cb[lo] <= g < inl_cb[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.inl_cb[mid] <= g) lo = mid;
    else hi = mid;
  }
  n = lo;
  c = g - p.inl_cb[lo];
}

__device__ __forceinline__ void chunk_of(const PrefillParams& p, int& n, int& c) {
  if (p.inl) {
    chunk_at(p, blockIdx.x, n, c);
  } else {
    c = blockIdx.x;
    n = blockIdx.y;
  }
}

__device__ __forceinline__ SeqInfo seq_info(const PrefillParams& p, int n) {
  SeqInfo s;
  long long b, e;
  if (p.inl) {
    b = p.inl_cu[n];
    e = p.inl_cu[n + 1];
  } else {
    b = read_dev(p.cu, n);
    e = read_dev(p.cu, n + 1);
  }
  if (b < 0 || e > p.T || e < b) { b = 0; e = 0; }  // inconsistent copy: treat as empty
  if (!p.inl && e > b &&
      (size_t)p.s.chunk_base[n] + (size_t)((e - b + kL - 1) / kL) > p.G) {
    b = 0;  // a device copy of cu_seqlens that disagrees with the host one
    e = 0;  // would overrun the scratch: treat the sequence as empty
  }
  s.begin = b;
  s.len = (int)(e - b);
  const int sl = p.slot_idx[n];
  s.slot = (sl >= 0 && sl < p.num_slots) ? sl : -1;
  s.init = p.has_init ? p.has_init[n] != 0 : true;
  return s;
}

// Raw (pre-conv) input of one channel at position `pos` relative to the
// start of a sequence: x rows for pos >= 0, the slot's conv window (whose
// last column is position -1) for negative pos, zero for a fresh sequence,
// past the end, or when `valid` is false.  The two base addresses are
// computed once per channel; a read is one select, one clamped index and one
// unconditional load (the value is selected afterwards), so that no
// conditional load forces a wait on every outstanding load.
template <typename Act, int K>
struct ChanReader {
  const char* xb;      // &x[begin][ch]
  const char* wb;      // &window[K][ch]: wb + pos * stride hits window row K + pos
  long long stride;    // bytes between consecutive positions (C elements)
  int len;
  bool init;

  __device__ __forceinline__ ChanReader(const PrefillParams& p, const SeqInfo& si, int ch) {
    using io = act_io<Act>;
    stride = (long long)p.C * io::bytes;
    xb = static_cast<const char*>(p.x) + ((long long)si.begin * p.C + ch) * io::bytes;
    wb = static_cast<const char*>(p.conv) + (size_t)si.slot * K * p.C * io::bytes +
         (long long)K * stride + (long long)ch * io::bytes;
    len = si.len;
    init = si.init;
  }

  // Unconverted element at `pos` (a readable address whatever `pos` is) and
  // whether it is part of the input; the caller applies both when it uses it,
  // so a prefetch leaves nothing to wait for.
  __device__ __forceinline__ typename act_io<Act>::raw_t fetch(int pos, bool valid, bool& use) const {
    const bool in_x = pos >= 0;
    use = valid & (in_x ? pos < len : (init & (pos >= -K)));
    const int pc = use ? pos : (in_x ? 0 : -1);
    const char* a = (in_x ? xb : wb) + (long long)pc * stride;
    return act_io<Act>::load_raw(a, 0);
  }

  __device__ __forceinline__ float operator()(int pos, bool valid = true) const {
    bool use;
    const float v = act_io<Act>::from_raw(fetch(pos, valid, use));
    return use ? v : 0.f;
  }

  // The 16 bytes starting at this channel (16 / element-size consecutive
  // channels) at `pos`.  Here `use` leaves out whether the slot holds an
  // initial window (the address must not wait for that flag): `win` marks a
  // window position, and the caller zeroes the bytes when !use, or when win
  // and the sequence starts fresh.
  __device__ __forceinline__ u32x4 fetch16(int pos, bool valid, bool& use, bool& win) const {
    const bool in_x = pos >= 0;
    use = valid & (in_x ? pos < len : pos >= -K);
    win = !in_x;
    const int pc = use ? pos : (in_x ? 0 : -1);
    const char* a = (in_x ? xb : wb) + (long long)pc * stride;
    return *reinterpret_cast<const u32x4*>(a);
  }
};

// 16 raw bytes as 16 / element-size floats.
template <typename Act>
__device__ __forceinline__ void unpack16(u32x4 r, float* f) {
  if constexpr (sizeof(Act) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(r[i] << 16);
      f[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
}

// Causal conv + SiLU of one 16-byte run of channels (V = 16 / element-size
// consecutive channels from ch, a multiple of V) over tokens i_off ..
// i_off+TPT-1 of the chunk starting at sequence position t0; tokens at or
// past nc give zero.  fetch() requests all TPT + K - 1 input runs and the
// weights (a handful of 16-byte loads instead of one load per element);
// finish() waits for them and computes, so other work can go in between.
template <typename Act, int K, int TPT>
struct ConvTile {
  static constexpr int V = 16 / sizeof(Act);
  u32x4 raw[TPT + K - 1];
  u32x4 wraw[K];
  uint32_t use;   // bit j: input run j is part of the input (window runs: if init)
  uint32_t win;   // bit j: input run j lies in the slot's conv window
  bool init;      // the window holds an initial state (applied in finish)

  __device__ __forceinline__ void fetch(const PrefillParams& p, const SeqInfo& si, int t0,
                                        int nc, int i_off, int ch) {
    const ChanReader<Act, K> rd(p, si, ch);
    use = 0;
    win = 0;
    init = si.init;
#pragma unroll
    for (int j = 0; j < TPT + K - 1; ++j) {
      const int r = i_off - (K - 1) + j;   // relative to the chunk start
      bool u, w;
      raw[j] = rd.fetch16(t0 + r, r < nc, u, w);
      use |= (uint32_t)u << j;
      win |= (uint32_t)w << j;
    }
    // weights of the V channels: V * K consecutive elements = K runs of 16 bytes
    const u32x4* wp = reinterpret_cast<const u32x4*>(static_cast<const char*>(p.conv_w) +
                                                     (size_t)ch * K * sizeof(Act));
#pragma unroll
    for (int k = 0; k < K; ++k) wraw[k] = wp[k];
  }

  __device__ __forceinline__ void finish(int nc, int i_off, float (&out)[TPT][V]) const {
    float wt[V * K];   // wt[v * K + k]
#pragma unroll
    for (int k = 0; k < K; ++k) unpack16<Act>(wraw[k], wt + k * V);
    const uint32_t eff = init ? use : use & ~win;
    float xs[TPT + K - 1][V];
#pragma unroll
    for (int j = 0; j < TPT + K - 1; ++j) {
      unpack16<Act>(raw[j], xs[j]);
#pragma unroll
      for (int v = 0; v < V; ++v) xs[j][v] = (eff >> j) & 1u ? xs[j][v] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < TPT; ++t)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) acc = fmaf(wt[v * K + k], xs[t + k][v], acc);
        out[t][v] = i_off + t < nc ? silu_fast(acc) : 0.f;
      }
  }
};

// --------------------------------------------------------------- MFMA helpers

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Lane layout of v_mfma_f32_16x16x32_bf16: A[i][k] at lane i + 16*(k/8),
// element k%8; B[k][j] at lane j + 16*(k/8), element k%8; D[i][j] at lane
// j + 16*(i/4), element i%4.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// (ah + al)(bh + bl) without the al*bl term, as three independent products
// accumulated separately so that consecutive k-steps of one tile do not wait
// on each other's passes; fold() adds the small terms first.
struct Acc3 {
  f32x4 hh, lh, hl;
};

__device__ __forceinline__ Acc3 acc3(f32x4 init) {
  return Acc3{init, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
}

__device__ __forceinline__ void mfma3(Acc3& c, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
  c.hh = mfma_bf16(ah, bh, c.hh);
  c.lh = mfma_bf16(al, bh, c.lh);
  c.hl = mfma_bf16(ah, bl, c.hl);
}

__device__ __forceinline__ f32x4 fold(const Acc3& c) { return (c.lh + c.hl) + c.hh; }

__device__ __forceinline__ void split_bf16(float v, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(v);
  lo = static_cast<__bf16>(v - static_cast<float>(hi));
}

// Eight consecutive f32 from LDS split into bf16 (hi, lo) fragments.
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h, l;
    split_bf16(v[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Fragment-major storage of an R x Kd bf16 MFMA A operand (R, Kd multiples
// of 16 and 32): tile (row block rb, k-step ks) is block rb * (Kd / 32) + ks
// of 64 lanes x 8 elements, lane li + 16 lk holding row 16 rb + li, columns
// 32 ks + 8 lk .. +7.  Element offset of (row, col), col a multiple of 4:
__device__ __forceinline__ size_t frag_at(size_t mat, int rows, int kd, int row, int col) {
  const size_t blk = mat * (size_t)((rows >> 4) * (kd >> 5)) + (row >> 4) * (kd >> 5) + (col >> 5);
  const int ln = (row & 15) + 16 * ((col & 31) >> 3);
  return (blk * 64 + ln) * 8 + (col & 7);
}

// Element offset of lane `lane` in block `blk` of a fragment-major operand.
__device__ __forceinline__ size_t frag_lane(size_t blk, int lane) {
  return (blk * 64 + lane) * 8;
}

// Four f32 split into bf16 (hi, lo) and stored as two 8-byte packs.
__device__ __forceinline__ void store_split4(__bf16* hi, __bf16* lo, f32x4 v) {
  bf16x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __bf16 a, b;
    split_bf16(v[e], a, b);
    h[e] = a;
    l[e] = b;
  }
  *reinterpret_cast<bf16x4*>(hi) = h;
  *reinterpret_cast<bf16x4*>(lo) = l;
}

// ------------------------------------------------------------------ 0. plan

// chunk_base[n] = sum over n' < n of ceil(len(n') / 64), chunk_base[N] = total.
// One workgroup of 1024 threads: per-thread partial sums over a contiguous
// range of sequences, then a wave64 shuffle scan and a scan of wave totals.
__device__ __forceinline__ int seq_chunks(const int32_t* cu, int n, long long T) {
  long long b = cu[n], e = cu[n + 1];
  if (b < 0 || e > T || e < b) return 0;
  return (int)((e - b + kL - 1) / kL);
}

__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t* cu, int N, long long T,
                                                            int32_t* chunk_base) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int per = (N + 1023) / 1024;
  const int n0 = tid * per, n1 = min(N, n0 + per);
  int local = 0;
  for (int n = n0; n < n1; ++n) local += seq_chunks(cu, n, T);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int v = wsum[w];
      wsum[w] = run;
      run += v;
    }
    chunk_base[N] = run;
  }
  __syncthreads();
  int run = wsum[wave] + incl - local;
  for (int n = n0; n < n1; ++n) {
    chunk_base[n] = run;
    run += seq_chunks(cu, n, T);
  }
}

// ------------------------------------------------------------------ 1. prep

// C[16x16] += A[16x16] B[16x16] on f32 MFMA, operands in LDS.
__device__ __forceinline__ f32x4 mm16(const float* A, int lda, const float* B, int ldb,
                                      f32x4 acc, int lane) {
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    acc = mfma_f32(A[li * lda + 4 * ks + lk], B[(4 * ks + lk) * ldb + li], acc);
  return acc;
}

// Tm = (I + A)^{-1} for strictly lower-triangular A [64][LDL] in LDS, blocked
// by 16: the four diagonal blocks by forward substitution (one lane per
// column), then wave jb < 4 walks down column block jb,
//   T_ib,jb = -T_ib,ib sum_{jb <= kb < ib} A_ib,kb T_kb,jb,   ib = jb+1 .. 3,
// reading only its own earlier blocks and the diagonal ones.  Called by every
// wave of the workgroup; ends with the lower blocks of the result in sT (the strictly
// upper blocks of sT are left as they are: the caller treats them as zero).
template <int LDL>
__device__ __forceinline__ void unit_lower_inverse(const float* sA, float* sT, float* sM, int tid) {
  const int lane = tid & 63, wave = wave_id();
  if (wave < 4 && lane < 16) {
    // column sweeps: once t_j is final, remove its term from every later row,
    // so the dependency chain is 15 steps long
    const int b0 = 16 * wave, c = lane;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = i == c ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j)
#pragma unroll
      for (int i = j + 1; i < 16; ++i) t[i] = fmaf(-sA[(b0 + i) * LDL + b0 + j], t[j], t[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[(b0 + i) * LDL + b0 + c] = t[i];
  }
  __syncthreads();
  const int li = lane & 15, lk = lane >> 4;
  const int jb = wave;              // waves 4 and up have no column block
  float* M = sM + (wave & 3) * 16 * 17;   // this wave's 16 x 16 staging tile
  for (int ib = jb + 1; ib < 4; ++ib) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb = jb; kb < ib; ++kb)
      acc = mm16(sA + 16 * ib * LDL + 16 * kb, LDL, sT + 16 * kb * LDL + 16 * jb, LDL, acc, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) M[(4 * lk + e) * 17 + li] = acc[e];
    acc = mm16(sT + 16 * ib * LDL + 16 * ib, LDL, M, 17, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(16 * ib + 4 * lk + e) * LDL + 16 * jb + li] = -acc[e];
  }
  __syncthreads();
}

// Both prep kernels depend on a chunk's own tokens only (WY form of the
// chunk, Gated DeltaNet paper, chunkwise training section):
//   q_hat, k_hat^T, K K^T, Q K^T            per K-head     (prefill_qk_kernel)
//   gamma = running sum of g, beta          per V-head     (prefill_wy_kernel)
//   A = strict_lower(beta_i e^{gamma_i - gamma_j} k_i.k_j), Tm = (I + A)^{-1}
//   P = lower(e^{gamma_i - gamma_j} q_i.k_j)
//   W = Tm diag(beta e^gamma) K,  U = Tm diag(beta) V
// so that the sequential pass only has V' = U - W S and the state update
// left.  Both keep their LDS near 40 KB and their registers under 170 so
// that three workgroups share a CU and hide each other's latencies.

// One workgroup per (chunk, sequence, K-head); wave w owns token block w.
// The conv output passes through one LDS tile: first the q rows, which each
// wave takes into registers as the MFMA A operand of its own token block (16
// tokens x D channels), then the k rows (f32) for the norms and the
// transposed k_hat^T reads, then the same k rows split once into bf16 (hi,
// lo) planes, from which the K K^T and Q K^T products read their operands
// directly.  One 35 KB tile instead of a q tile beside the k tile leaves room
// for three workgroups per CU.
template <typename Act, int D, int K>
__global__ __launch_bounds__(kNT, 3) void prefill_qk_kernel(PrefillParams p) {
  constexpr int LDD = D + 4, NTL = kL / 16, NKS = D / 32;
  constexpr int LDH = D + 8;   // row length of the bf16 planes
  constexpr int XB = kL * LDD * 4, HB = 2 * kL * LDH * 2;
  static_assert(NTL == kNW, "one token block per wave");
  // q rows, then k rows (f32, unnormalized); then the k rows as hi and lo planes
  __shared__ __attribute__((aligned(16))) unsigned char sBuf[XB > HB ? XB : HB];
  float* sX = reinterpret_cast<float*>(sBuf);
  __bf16* sKh = reinterpret_cast<__bf16*>(sBuf);
  __bf16* sKl = sKh + kL * LDH;
  __shared__ float sRq[kL], sRk[kL];

  int n, c;
  chunk_of(p, n, c);
  const int m = blockIdx.z;
  const SeqInfo si = seq_info(p, n);
  const int t0 = c * kL;
  if (si.slot < 0 || t0 >= si.len) return;
  const int nc = min(kL, si.len - t0);
  const size_t gk = (chunk_base_of(p, n) + c) * p.Hk + m;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 15, lk = lane >> 4;

  // conv + SiLU of q_m and k_m: thread = (16-byte channel run, run of tokens)
  constexpr int V = 16 / sizeof(Act), G = 2 * D / V, TPT = kL * G / kNT;
  static_assert(kNT % G == 0 && TPT >= 1, "q/k conv split");
  const int grp = tid % G, i_off = (tid / G) * TPT;
  const int c0 = grp * V;                      // 0 .. 2D-1: q then k
  const bool isq = c0 < D;
  const int dcol = isq ? c0 : c0 - D;
  float out[TPT][V];
  {
    const int ch = isq ? m * D + c0 : (p.Hk + m) * D + (c0 - D);
    ConvTile<Act, K, TPT> ct;
    ct.fetch(p, si, t0, nc, i_off, ch);
    ct.finish(nc, i_off, out);
  }
  auto put = [&]() {
#pragma unroll
    for (int t = 0; t < TPT; ++t)
#pragma unroll
      for (int v = 0; v < V; v += 4)
        *reinterpret_cast<f32x4*>(sX + (i_off + t) * LDD + dcol + v) =
            f32x4{out[t][v], out[t][v + 1], out[t][v + 2], out[t][v + 3]};
  };
  // q rows -> A operand of this wave's token block: token 16 wave + li,
  // channels 32 ks + 8 lk .. +7
  if (isq) put();
  __syncthreads();
  float qa[NKS][8];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sX + (16 * wave + li) * LDD + 32 * ks + 8 * lk + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) qa[ks][4 * hf + e] = v[e];
    }
  __syncthreads();
  if (!isq) put();
  __syncthreads();
  // l2 norms as per-row factors (q's includes the 1/sqrt(dk) scale), applied
  // where the rows are used: q over the four lanes of a token, k over PARTS
  // lanes per row of the tile
  {
    float sq = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) sq = fmaf(qa[ks][e], qa[ks][e], sq);
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    if (lk == 0) sRq[16 * wave + li] = p.scale / sqrtf(sq + p.l2eps);
    constexpr int PARTS = kNT / kL, QD = D / PARTS;
    const int i = tid / PARTS, part = tid % PARTS;
    float sk = 0.f;
#pragma unroll
    for (int d = part * QD; d < (part + 1) * QD; ++d) {
      const float kv = sX[i * LDD + d];
      sk = fmaf(kv, kv, sk);
    }
#pragma unroll
    for (int off = 1; off < PARTS; off <<= 1) sk += __shfl_xor(sk, off, 64);
    if (part == 0) sRk[i] = 1.0f / sqrtf(sk + p.l2eps);
  }
  __syncthreads();
  // q_hat rows as bf16 (hi, lo) fragments, straight from the registers (the
  // wave's lane is the fragment lane of block (token block, ks)); the raw q
  // split once for the Q K^T products
  bf16x8 qh[NKS], ql[NKS];
  {
    const float rq = sRq[16 * wave + li];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = qa[ks][e] * rq;
      bf16x8 h, l;
      split8(v, h, l);
      const size_t at = frag_lane(gk * (NTL * NKS) + wave * NKS + ks, lane);
      *reinterpret_cast<bf16x8*>(p.s.qh[0] + at) = h;
      if (!p.o_bf16) *reinterpret_cast<bf16x8*>(p.s.qh[1] + at) = l;   // (read by 3-pass outputs only)
      split8(qa[ks], qh[ks], ql[ks]);
    }
  }
  // k_hat^T as bf16 (hi, lo) fragments: the lanes of a wave take consecutive
  // channels d, so the column reads of the tile fall in distinct banks
  for (int u = tid; u < D * (kL / 8); u += kNT) {
    const int d = u % D, i0 = 8 * (u / D);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = sX[(i0 + e) * LDD + d] * sRk[i0 + e];
    bf16x8 h, l;
    split8(v, h, l);
    const size_t at = frag_at(gk, D, kL, d, i0);
    *reinterpret_cast<bf16x8*>(p.s.kt[0] + at) = h;
    *reinterpret_cast<bf16x8*>(p.s.kt[1] + at) = l;
  }
  // the raw k rows split once into the hi and lo planes, in place: each
  // thread takes SH consecutive values of one row, then writes them back split
  // after every read of the f32 tile is done
  {
    constexpr int SH = kL * D / kNT, PER = D / SH;
    static_assert(SH % 8 == 0 && PER * SH == D, "plane split");
    const int r = tid / PER, c0 = (tid % PER) * SH;
    bf16x8 h[SH / 8], l[SH / 8];
#pragma unroll
    for (int j = 0; j < SH / 8; ++j) split8(sX + r * LDD + c0 + 8 * j, h[j], l[j]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SH / 8; ++j) {
      *reinterpret_cast<bf16x8*>(sKh + r * LDH + c0 + 8 * j) = h[j];
      *reinterpret_cast<bf16x8*>(sKl + r * LDH + c0 + 8 * j) = l[j];
    }
    __syncthreads();
  }
  // K K^T and Q K^T, lower block triangle, 3-pass bf16, rows scaled by the
  // norm factors, out as f32 [64][64] (the strictly upper blocks are not
  // written; their readers select them away).  Wave w takes the Q K^T tiles
  // of its own token block (w + 1 of them) and 4 - w of the K K^T tiles, five
  // tiles per wave.
  float* gG = p.s.gq + gk * 2 * kL * kL;
  auto tile = [&](bool isG, int I, int J) {
    Acc3 acc = acc3(f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int bo = (16 * J + li) * LDH + 32 * ks + 8 * lk;
      const bf16x8 bh = ld8(sKh + bo), bl = ld8(sKl + bo);
      if (isG) {
        const int ao = (16 * I + li) * LDH + 32 * ks + 8 * lk;
        mfma3(acc, ld8(sKh + ao), ld8(sKl + ao), bh, bl);
      } else {
        mfma3(acc, qh[ks], ql[ks], bh, bl);
      }
    }
    const f32x4 r = fold(acc);
    float* dst = gG + (isG ? 0 : kL * kL);
    const float* ra = isG ? sRk : sRq;
    const float rj = sRk[16 * J + li];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * I + 4 * lk + e;
      dst[i * kL + 16 * J + li] = r[e] * ra[i] * rj;
    }
  };
  for (int J = 0; J <= wave; ++J) tile(false, wave, J);
  const int first = 4 * wave - wave * (wave - 1) / 2;   // K K^T tiles first .. first + 3 - wave
  for (int t = first; t < first + NTL - wave; ++t) {
    int I = 0, rem = t;
    while (rem > I) { rem -= I + 1; ++I; }
    tile(true, I, rem);
  }
}

// One workgroup per (chunk, V-head).  W's row factor beta_j e^{gamma_j} is
// split between the two sides of W^T = (K^T diag(e^gamma)) (Tm diag(beta))^T:
// e^gamma scales the k_hat^T fragments from the q/k kernel in registers, so
// W and U share the one LDS tile Tm diag(beta).  The v conv is computed
// straight into the B-operand registers of U (each lane: one channel, eight
// consecutive tokens), so v never passes through LDS, and the split Tm
// diag(beta) takes the place of A once the inverse is done: 40 KB of LDS.
template <typename Act, int D, int K>
__global__ __launch_bounds__(kNT, 3) void prefill_wy_kernel(PrefillParams p) {
  using io = act_io<Act>;
  constexpr int LDL = kL + 4, NTL = kL / 16, NDB = D / 16;
  constexpr int DBW = (NDB + kNW - 1) / kNW;   // column blocks per wave
  constexpr int LDH = kL + 8;   // bf16 row length of the split Tm tiles (16-byte rows)
  // region 0 holds A (f32), then the split Tm diag(beta) (bf16 hi, lo);
  // region 1 holds Tm (f32)
  constexpr int R0 = kL * LDL * 4 > 2 * kL * LDH * 2 ? kL * LDL * 4 : 2 * kL * LDH * 2;
  __shared__ __attribute__((aligned(16))) unsigned char sAT[R0 + kL * LDL * 4];
  __shared__ __attribute__((aligned(16))) float sM[4 * 16 * 17];    // the inverse's staging tiles
  __shared__ float sGam[kL], sBeta[kL], sEg[kL];
  float* sA = reinterpret_cast<float*>(sAT);
  float* sT = reinterpret_cast<float*>(sAT + R0);
  __bf16* sTb0 = reinterpret_cast<__bf16*>(sAT);   // Tm diag(beta) hi, lo: in A's place
  __bf16* sTb1 = sTb0 + kL * LDH;

  // Block x -> unit (chunk, K-head) = (x / (8 r)) * 8 + x % 8 and V-head
  // m r + (x / 8) % r: the r workgroups of a unit get ids 8 apart, so they
  // are dispatched together onto one XCD and read the unit's K K^T, Q K^T
  // and k_hat^T fragments through one L2.  Chunks run along x (all real
  // chunks when the prefix travels with the launch, else one sequence's
  // chunk slots per y).
  const int per = 8 * p.r, xg = blockIdx.x / per, xr = blockIdx.x - xg * per;
  const int unit = xg * 8 + (xr & 7);
  const int cx = p.inl ? p.inl_cb[p.N] : p.max_chunks;
  if (unit >= cx * p.Hk) return;
  const int m = unit % p.Hk;
  const int h = m * p.r + (xr >> 3);
  int n, c;
  if (p.inl) {
    chunk_at(p, unit / p.Hk, n, c);
  } else {
    n = blockIdx.y;
    c = unit / p.Hk;
  }
  const SeqInfo si = seq_info(p, n);
  const int t0 = c * kL;
  if (si.slot < 0 || t0 >= si.len) return;
  const int nc = min(kL, si.len - t0);
  const long long tok0 = si.begin + t0;
  const size_t g = chunk_base_of(p, n) + c;
  const size_t gh = g * p.Hv + h, gk = g * p.Hk + m;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 15, lk = lane >> 4;

  // K K^T and Q K^T rows of this thread's A/P runs and the gate inputs
  // (wave 0) are requested first
  constexpr int APR = kL * (kL / 8) / kNT;   // A/P runs per thread
  static_assert(kL * (kL / 8) % kNT == 0, "A/P split");
  const float* gG = p.s.gq + gk * 2 * kL * kL;
  const float* gQK = gG + kL * kL;
  f32x4 kkr[APR][2], qkr[APR][2];
#pragma unroll
  for (int q = 0; q < APR; ++q) {
    const int u = tid + q * kNT, i = u / (kL / 8), j0 = 8 * (u - i * (kL / 8));
    // runs wholly above the diagonal are never used: they read the row's
    // first run instead (a line fetched anyway), so the upper half of the
    // tiles costs no memory traffic
    const int jr = j0 <= i ? j0 : 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      kkr[q][hf] = *reinterpret_cast<const f32x4*>(gG + i * kL + jr + 4 * hf);
      qkr[q][hf] = *reinterpret_cast<const f32x4*>(gQK + i * kL + jr + 4 * hf);
    }
  }
  float a_in = 0.f, b_in = 0.f, alog = 0.f, dtb = 0.f;
  if (wave == 0) {
    const long long tk = tok0 + min(lane, nc - 1);
    a_in = io::load(p.a, (size_t)tk * p.Hv + h);
    b_in = io::load(p.b, (size_t)tk * p.Hv + h);
    alog = p.A_log[h];
    dtb = p.dt_bias[h];
  }
  // gates: running sum gamma, beta, and e^gamma (the K side of W's factor)
  if (wave == 0) {
    float gv = 0.f, bv = 0.f;
    if (lane < nc) gates(alog, dtb, a_in, b_in, gv, bv);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(gv, off, 64);
      if (lane >= off) gv += y;
    }
    sGam[lane] = gv;
    sBeta[lane] = bv;
    sEg[lane] = expf(gv);
    p.s.gam[gh * kL + lane] = gv;
  }
  __syncthreads();
  // A (for the inverse; only its lower triangle is read) and P (written out
  // as fragments), sharing one decay e^{gamma_i - gamma_j} per element
#pragma unroll
  for (int q = 0; q < APR; ++q) {
    const int u = tid + q * kNT, i = u / (kL / 8), j0 = 8 * (u - i * (kL / 8));
    const float gi = sGam[i], bi = sBeta[i];
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // selects, not products with a zero mask: the strictly upper blocks
      // of K K^T and Q K^T are never written and may hold any bits
      const int j = j0 + e;
      const float kk = kkr[q][e >> 2][e & 3], qk = qkr[q][e >> 2][e & 3];
      const float dec = j <= i ? __expf(gi - sGam[j]) : 0.f;
      sA[i * LDL + j] = j < i ? bi * dec * kk : 0.f;
      v[e] = j <= i ? dec * qk : 0.f;
    }
    bf16x8 h8, l8;
    split8(v, h8, l8);
    const size_t at = frag_at(gh, kL, kL, i, j0);
    *reinterpret_cast<bf16x8*>(p.s.pm[0] + at) = h8;
    if (!p.o_bf16) *reinterpret_cast<bf16x8*>(p.s.pm[1] + at) = l8;   // (read by 3-pass outputs only)
  }
  // v conv inputs in the B-operand layout of U: for column block db = wave +
  // kNW it and k-step ks, lane li + 16 lk takes channel 16 db + li at tokens
  // 32 ks + 8 lk .. +7, i.e. the K - 1 + 8 raw inputs from 32 ks + 8 lk - (K - 1)
  constexpr int VR = 8 + K - 1;                // raw inputs per (block, k-step)
  typename act_io<Act>::raw_t vraw[DBW][2][VR], vwr[DBW][K];
  uint32_t vuse[DBW][2];
#pragma unroll
  for (int it = 0; it < DBW; ++it) {
    const int db = min(wave + kNW * it, NDB - 1);
    const int ch = 2 * p.Hk * D + h * D + 16 * db + li;
    const ChanReader<Act, K> rd(p, si, ch);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      vuse[it][ks] = 0;
#pragma unroll
      for (int j = 0; j < VR; ++j) {
        const int r = 32 * ks + 8 * lk - (K - 1) + j;   // relative to the chunk start
        bool u;
        vraw[it][ks][j] = rd.fetch(t0 + r, r < nc, u);
        vuse[it][ks] |= (uint32_t)u << j;
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) vwr[it][k] = io::load_raw(p.conv_w, (size_t)ch * K + k);
  }
  // k_hat^T fragments of this wave's W/U column blocks db = wave + kNW it
  // (the A operand of W^T, from the q/k kernel).  These and the v conv
  // inputs above are requested only here, once A and P are formed, so their
  // latency passes under the inverse and their registers are not held
  // beside the K K^T / Q K^T rows (148 registers instead of 168)
  bf16x8 kth[DBW][2], ktl[DBW][2];
#pragma unroll
  for (int it = 0; it < DBW; ++it) {
    const int db = min(wave + kNW * it, NDB - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const size_t at = frag_lane((gk * NDB + db) * 2 + ks, lane);
      kth[it][ks] = ld8(p.s.kt[0] + at);
      ktl[it][ks] = ld8(p.s.kt[1] + at);
    }
  }
  __syncthreads();
  // (the inverse ends with a barrier)
  unit_lower_inverse<LDL>(sA, sT, sM, tid);
  // v conv + SiLU (tokens at or past nc give zero), held as U's B operand
  float vo[DBW][2][8];
#pragma unroll
  for (int it = 0; it < DBW; ++it) {
    float w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = io::from_raw(vwr[it][k]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float xs[VR];
#pragma unroll
      for (int j = 0; j < VR; ++j)
        xs[j] = (vuse[it][ks] >> j) & 1u ? io::from_raw(vraw[it][ks][j]) : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) acc = fmaf(w[k], xs[e + k], acc);
        vo[it][ks][e] = 32 * ks + 8 * lk + e < nc ? silu_fast(acc) : 0.f;
      }
    }
  }
  // Tm diag(beta), split (strictly upper blocks zero)
  for (int u = tid; u < kL * (kL / 8); u += kNT) {
    const int i = u / (kL / 8), j0 = 8 * (u - i * (kL / 8));
    const bool upper = (j0 >> 4) > (i >> 4);
    float vb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vb[e] = upper ? 0.f : sT[i * LDL + j0 + e] * sBeta[j0 + e];
    bf16x8 h8, l8;
    split8(vb, h8, l8);
    *reinterpret_cast<bf16x8*>(sTb0 + i * LDH + j0) = h8;
    *reinterpret_cast<bf16x8*>(sTb1 + i * LDH + j0) = l8;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < DBW; ++it) {
    const int db = wave + kNW * it;
    if (db >= NDB) break;   // uniform: fewer column blocks than waves
    // k_hat^T rows 16 db + li times e^{gamma_j} at token j = 32 ks + 8 lk + e,
    // split again (A operand of W^T)
    bf16x8 kh[2], kl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        kv[e] = ((float)kth[it][ks][e] + (float)ktl[it][ks][e]) * sEg[32 * ks + 8 * lk + e];
      split8(kv, kh[ks], kl[ks]);
    }
    // v of channel d at the lane's tokens, split (B operand of U)
    bf16x8 vh[2], vl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) split8(vo[it][ks], vh[ks], vl[ks]);
#pragma unroll
    for (int tb = 0; tb < NTL; ++tb) {
      // rows 16 tb + li of Tm diag(beta): B operand of W^T and A operand of U
      bf16x8 bh[2], bl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int o = (16 * tb + li) * LDH + 32 * ks + 8 * lk;
        bh[ks] = ld8(sTb0 + o);
        bl[ks] = ld8(sTb1 + o);
      }
      Acc3 aw = acc3(f32x4{0.f, 0.f, 0.f, 0.f});   // W^T: rows d, columns token
      Acc3 au = acc3(f32x4{0.f, 0.f, 0.f, 0.f});   // U: rows token, columns d
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        mfma3(aw, kh[ks], kl[ks], bh[ks], bl[ks]);
        mfma3(au, bh[ks], bl[ks], vh[ks], vl[ks]);
      }
      const f32x4 wt = -fold(aw);   // -W[token 16 tb + li][d 16 db + 4 lk + e]
      const size_t wo = frag_at(gh, kL, D, 16 * tb + li, 16 * db + 4 * lk);
      store_split4(p.s.w[0] + wo, p.s.w[1] + wo, wt);
      // U tile in the accumulator layout of the state kernel: block
      // (d block db, token block tb), lane li + 16 lk
      *reinterpret_cast<f32x4*>(p.s.ut + (((gh * NDB + db) * NTL + tb) * 64 + lane) * 4) = fold(au);
    }
  }
}

// ------------------------------------------------------------------ 2. state

// Recurrence waves of the state kernel: eight for a 16-column tile (one
// state row block each, half of them idle in the first phase), four
// otherwise (two row blocks each); four output waves beside them.
template <int NCB> constexpr int state_rec_waves() { return NCB == 1 ? 8 : 4; }
template <int NCB> constexpr int state_threads() { return 64 * (state_rec_waves<NCB>() + 4); }

// Compile-time wave role of the state kernel's chunk loop: 0 recurrence
// waves that also form V' (token block = wave), 1 recurrence waves that only
// update their state row blocks, 2 output waves.
template <int R> struct WaveRole { static constexpr int value = R; };

// Operands of one chunk held in registers by one wave of the state kernel;
// the next chunk's are fetched into the same registers right after their
// last use.  The same registers serve every wave role:
//   recurrence waves   fa = -W rows (those that form V'), fb = k_hat^T rows
//                      of the owned state row blocks, u = U tiles
//   output waves       fa = q_hat rows, fb[0] = P rows
template <int NKS, int RBW, int NCB>
struct ChunkOps {
  bf16x8 fa[NKS][2];
  bf16x8 fb[RBW][2][2];   // [row block][k-step][hi, lo]
  f32x4 u[NCB];           // token rows i0 .. i0+3 of column 16 cb + li
  f32x4 gam;              // gamma at rows i0 .. i0+3
  float glast;            // gamma at the chunk's last token
};

// One workgroup per (sequence, V-head, 16 NCB state columns), one pass over
// the sequence's chunks (chunk recurrence of the WY form: V' = U - W S,
// S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) V', O = e^gamma Q S + P V').
// The first NRW waves carry the recurrence; the last four compute the
// chunk's outputs from the same S and V' tiles in LDS, beside it, so the
// serial chain per chunk is two contractions and two barriers.  Every
// operand fetch is one contiguous 1 KB fragment block per wave.
template <typename Act, int D, int K, int NCB, bool OB>
__global__ __launch_bounds__(state_threads<NCB>()) void prefill_state_kernel(PrefillParams p) {
  using io = act_io<Act>;
  constexpr int NRW = state_rec_waves<NCB>();
  constexpr int NTH = state_threads<NCB>();
  constexpr int DVT = 16 * NCB;        // state columns of the workgroup
  constexpr int NKS = D / 32;          // k-steps over d
  constexpr int NRB = D / 16;          // 16-row blocks of the state tile
  constexpr int RBW = (NRB + NRW - 1) / NRW;   // state row blocks per recurrence wave
  constexpr int LS = D + 8;            // row length of the transposed state [j][d]
  constexpr int LR = kL + 8;           // row length of [j][token] tiles
  __shared__ __attribute__((aligned(16))) __bf16 sS[2][DVT * LS];   // S_c, B operand
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][DVT * LR];   // V'
  __shared__ __attribute__((aligned(16))) __bf16 sD[2][DVT * LR];   // e^{gamma_L - gamma} V'
  // bf16 outputs: the output waves leave a chunk's O here and, during the
  // next chunk's first phase, where they wait on the recurrence, write it
  // out with 16-byte stores (with eight recurrence waves the four that are
  // idle in that phase do it instead)
  constexpr bool STAGE_O = OB;
  constexpr int FLUSH_ROLE = NRW == 8 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) __bf16 sO[STAGE_O ? kL * DVT : 8];

  // Workgroup id -> (sequence, V-head, column tile): the r * tiles
  // workgroups of one (sequence, K-head) get ids 8 apart, so they land on one
  // XCD and are dispatched together; the chunk operands of the K-head and of
  // its V-heads then come from HBM once per XCD L2 rather than once per tile.
  const int tiles = D / DVT, per = p.r * tiles;
  const int grp = blockIdx.x / (8 * per), rem = blockIdx.x - grp * 8 * per;
  const int unit = grp * 8 + (rem & 7), k = rem >> 3;
  if (unit >= p.N * p.Hk) return;
  const int nu = unit / p.Hk, m = unit - nu * p.Hk;
  const int n = p.inl ? p.inl_order[nu] : nu;
  const int h = m * p.r + k / tiles, col0 = (k % tiles) * DVT;
  const SeqInfo si = seq_info(p, n);
  if (si.slot < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int li = lane & 15, lk = lane >> 4;
  const bool rec = wave < NRW;                 // recurrence wave
  // token-row block (and first state row block): the wave's index within its role
  const int w4 = NRW == 4 ? (wave & 3) : (rec ? wave : wave - NRW);
  const int i0 = 16 * (w4 & 3) + 4 * lk;       // first of this lane's four token rows
  float* Sg = p.rec + ((size_t)si.slot * p.Hv + h) * D * D;
  const size_t cbase = si.len > 0 ? chunk_base_of(p, n) : 0;
  const int nchunks = (si.len + kL - 1) / kL;

  // S_0: every load of a recurrence wave is issued before any is used (row
  // blocks past the state are clamped and dropped), and a slot without an
  // initial state is masked to zero bit by bit.  A branch or a select there
  // would make the compiler test has_init first and wait for each block's
  // loads before issuing the next.
  f32x4 S[RBW][NCB];
#pragma unroll
  for (int q = 0; q < RBW; ++q)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) S[q][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (rec) {
    float v[RBW][NCB][4];
#pragma unroll
    for (int q = 0; q < RBW; ++q) {
      const int rb = min(w4 + NRW * q, NRB - 1);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[q][cb][e] = Sg[(size_t)(16 * rb + 4 * lk + e) * D + col0 + 16 * cb + li];
    }
    const unsigned keep_bits = si.init ? ~0u : 0u;
#pragma unroll
    for (int q = 0; q < RBW; ++q)
      if (w4 + NRW * q < NRB)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            S[q][cb][e] = __uint_as_float(__float_as_uint(v[q][cb][e]) & keep_bits);
  }

  // S_0 into LDS as hi/lo bf16, columns major
  if (rec)
#pragma unroll
    for (int q = 0; q < RBW; ++q) {
      const int rb = w4 + NRW * q;
      if (rb < NRB)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            __bf16 hi, lo;
            split_bf16(S[q][cb][e], hi, lo);
            sS[0][(16 * cb + li) * LS + 16 * rb + 4 * lk + e] = hi;
            sS[1][(16 * cb + li) * LS + 16 * rb + 4 * lk + e] = lo;
          }
    }

  // The chunk loop, instantiated once per wave role (REC: the recurrence
  // waves).  With the role a compile-time constant the loop holds no role
  // branch, so the registers a role carries from chunk to chunk are never
  // merged with the other role's; such a merge copies just-loaded registers
  // and so waits for their loads at once.  Both instantiations pass the same
  // barriers in the same order.  Loads are unconditional within a role
  // (chunk index clamped), so the prefetch of chunk c+1 never introduces a
  // branch and its wait.
  const auto chunk_loop = [&](auto role) {
    constexpr int ROLE = decltype(role)::value;
    constexpr bool REC = ROLE < 2;       // carries state row blocks
    constexpr bool VP = ROLE == 0;       // forms V' in the first phase
    ChunkOps<NKS, RBW, NCB> ops;
    auto load_fa = [&](int c) {
      if constexpr (ROLE == 1) return;   // no first-phase product
      const size_t mat = REC ? (cbase + c) * p.Hv + h : (cbase + c) * p.Hk + m;
      const __bf16* hi = REC ? p.s.w[0] : p.s.qh[0];
      const __bf16* lo = REC ? p.s.w[1] : p.s.qh[1];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const size_t at = frag_lane(mat * (4 * NKS) + w4 * NKS + ks, lane);
        ops.fa[ks][0] = ld8(hi + at);
        if constexpr (REC || !OB) ops.fa[ks][1] = ld8(lo + at);
      }
    };
    auto load_fb = [&](int c) {
      const __bf16* hi = REC ? p.s.kt[0] : p.s.pm[0];
      const __bf16* lo = REC ? p.s.kt[1] : p.s.pm[1];
#pragma unroll
      for (int q = 0; q < (REC ? RBW : 1); ++q) {   // output waves need one P row block
        const int rb = min(w4 + NRW * q, NRB - 1);
        const size_t blk0 = REC ? (((cbase + c) * p.Hk + m) * NRB + rb) * 2
                                : (((cbase + c) * p.Hv + h) * 4 + w4) * 2;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const size_t at = frag_lane(blk0 + ks, lane);
          ops.fb[q][ks][0] = ld8(hi + at);
          if constexpr (REC || !OB) ops.fb[q][ks][1] = ld8(lo + at);
        }
      }
    };
    auto load_misc = [&](int c) {
      const int nc = min(kL, si.len - c * kL);
      const size_t gh = (cbase + c) * p.Hv + h;
      if constexpr (VP)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          ops.u[cb] = *reinterpret_cast<const f32x4*>(
              p.s.ut + (((gh * NRB + col0 / 16 + cb) * 4 + w4) * 64 + lane) * 4);
      if constexpr (ROLE != 1) ops.gam = *reinterpret_cast<const f32x4*>(p.s.gam + gh * kL + i0);
      ops.glast = p.s.gam[gh * kL + nc - 1];
    };

    // chunk c-1's staged outputs to global memory, written by the FLUSH_ROLE waves
    long long otok0 = 0;
    int onc = 0;
    auto flush_o = [&]() {
      constexpr int PR = DVT / 8;                 // 16-byte pieces per token row
      const int first = (NRW == 8 ? wave - 4 : wave - NRW) * 64 + lane;
      const auto put = [&](int q) {
        const int i = q / PR, part = q % PR;
        if (i < onc)
          *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(p.obuf) +
                                     ((size_t)(otok0 + i) * p.Hv + h) * D + col0 + 8 * part) =
              *reinterpret_cast<const bf16x8*>(&sO[i * DVT + 8 * part]);
      };
      // four flushing waves: one piece per lane up to 32 columns (measured
      // faster than the loop there), a loop over the pieces at 64
      if constexpr (kL * PR <= 256) put(first);
      else
        for (int q = first; q < kL * PR; q += 256) put(q);
    };

    if (nchunks > 0) {  // same issue order as in the loop (see its waits)
      load_misc(0);
      load_fa(0);
      load_fb(0);
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
      const int t0 = c * kL, nc = min(kL, si.len - t0);
      const long long tok0 = si.begin + t0;
      const int cn = min(c + 1, nchunks - 1);  // chunk whose operands are prefetched
      // U and gamma are needed first: take them and refetch for the next
      // chunk at once, so their loads are the oldest outstanding ones a
      // chunk later
      f32x4 u[NCB];
      f32x4 gam = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (VP)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) u[cb] = ops.u[cb];
      if constexpr (ROLE != 1) gam = ops.gam;
      const float glast = ops.glast;
      load_misc(cn);
      if constexpr (STAGE_O && ROLE == FLUSH_ROLE) {
        if (c > 0) flush_o();
        otok0 = tok0;
        onc = nc;
      }
      // phase 1: V' = U - W S_c (recurrence waves) / Y = Q S_c (output waves)
      f32x4 O[NCB];
#pragma unroll
      for (int cb = 0; cb < (ROLE == 1 ? 0 : NCB); ++cb) {
        f32x4 r1;
        if constexpr (!REC && OB) {
          // output-only product, single pass (bf16 output path)
          r1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            r1 = mfma_bf16(ops.fa[ks][0], ld8(&sS[0][(16 * cb + li) * LS + 32 * ks + 8 * lk]), r1);
        } else {
          Acc3 acc = acc3(VP ? u[cb] : f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int bo = (16 * cb + li) * LS + 32 * ks + 8 * lk;
            mfma3(acc, ops.fa[ks][0], ops.fa[ks][1], ld8(&sS[0][bo]), ld8(&sS[1][bo]));
          }
          r1 = fold(acc);
        }
        if constexpr (REC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * cb + li, i = i0 + e;
            __bf16 hi, lo;
            split_bf16(r1[e], hi, lo);
            sV[0][j * LR + i] = hi;
            sV[1][j * LR + i] = lo;
            split_bf16(__expf(glast - gam[e]) * r1[e], hi, lo);
            sD[0][j * LR + i] = hi;
            sD[1][j * LR + i] = lo;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) O[cb][e] = __expf(gam[e]) * r1[e];
        }
      }
      load_fa(cn);
      __syncthreads();  // V' is in LDS; every read of S_c is done
      if constexpr (REC) {
        // phase 2: S <- e^{gamma_L} S + K^T (e^{gamma_L - gamma} V')
        const float egl = __expf(glast);
#pragma unroll
        for (int q = 0; q < RBW; ++q) {
          const int rb = w4 + NRW * q;
          if (rb < NRB)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              Acc3 as = acc3(S[q][cb] * egl);
#pragma unroll
              for (int ks = 0; ks < 2; ++ks) {
                const int bo = (16 * cb + li) * LR + 32 * ks + 8 * lk;
                mfma3(as, ops.fb[q][ks][0], ops.fb[q][ks][1], ld8(&sD[0][bo]), ld8(&sD[1][bo]));
              }
              S[q][cb] = fold(as);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                __bf16 hi, lo;
                split_bf16(S[q][cb][e], hi, lo);
                sS[0][(16 * cb + li) * LS + 16 * rb + 4 * lk + e] = hi;
                sS[1][(16 * cb + li) * LS + 16 * rb + 4 * lk + e] = lo;
              }
            }
        }
      } else {
        // O += P V', stored as the pre-norm output
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          f32x4 o;
          if constexpr (OB) {
            o = O[cb];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              o = mfma_bf16(ops.fb[0][ks][0], ld8(&sV[0][(16 * cb + li) * LR + 32 * ks + 8 * lk]), o);
          } else {
            Acc3 ao = acc3(O[cb]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const int bo = (16 * cb + li) * LR + 32 * ks + 8 * lk;
              mfma3(ao, ops.fb[0][ks][0], ops.fb[0][ks][1], ld8(&sV[0][bo]), ld8(&sV[1][bo]));
            }
            o = fold(ao);
          }
          if constexpr (STAGE_O) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sO[(i0 + e) * DVT + 16 * cb + li] = static_cast<__bf16>(o[e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = i0 + e;
              const size_t at = ((size_t)(tok0 + i) * p.Hv + h) * D + col0 + 16 * cb + li;
              if (i < nc) {
                if constexpr (OB) reinterpret_cast<__bf16*>(p.obuf)[at] = static_cast<__bf16>(o[e]);
                else p.obuf[at] = o[e];
              }
            }
          }
        }
      }
      load_fb(cn);
      __syncthreads();  // S_{c+1} is in LDS; every read of V' is done
    }
    if constexpr (STAGE_O && ROLE == FLUSH_ROLE)
      if (nchunks > 0) flush_o();   // the last chunk's outputs (after its closing barrier)
  };
  if (!rec) {
    chunk_loop(WaveRole<2>{});
  } else if constexpr (NRW == 4) {
    chunk_loop(WaveRole<0>{});
  } else {
    if (wave < 4)
      chunk_loop(WaveRole<0>{});
    else
      chunk_loop(WaveRole<1>{});
  }

  if (rec)
#pragma unroll
    for (int q = 0; q < RBW; ++q) {
      const int rb = w4 + NRW * q;
      if (rb < NRB)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Sg[(size_t)(16 * rb + 4 * lk + e) * D + col0 + 16 * cb + li] = S[q][cb][e];
    }

  // Final conv window = the last K raw inputs of [window ; tokens], for this
  // tile's v channels, plus the q/k channels of K-head m from tile 0 of its
  // first V-head.  No other workgroup reads these channels of the window
  // (the prep kernel, an earlier launch, read all of them).
  {
    const bool qk = col0 == 0 && h % p.r == 0;
    const int nch = DVT + (qk ? 2 * D : 0);
    const int vbase = 2 * p.Hk * D + h * D + col0;
    void* win = static_cast<char*>(p.conv) + (size_t)si.slot * K * p.C * io::bytes;
    for (int e = tid; e < nch; e += NTH) {
      const int ch = e < DVT ? vbase + e
                   : e < DVT + D ? m * D + (e - DVT)
                                 : (p.Hk + m) * D + (e - DVT - D);
      const ChanReader<Act, K> rd(p, si, ch);
      float vals[K];
#pragma unroll
      for (int j = 0; j < K; ++j) vals[j] = rd(si.len - K + j);
#pragma unroll
      for (int j = 0; j < K; ++j) io::store(win, (size_t)j * p.C + ch, vals[j]);
    }
  }
}

// ------------------------------------------------------------------ 3. norm

// 256 threads = ROWS token rows x LPR lanes; a lane owns 8 consecutive values
// of each of the chunk's rows r, r + ROWS, ... (16-byte runs of z and y in
// bf16, 32 bytes of the f32 pre-norm output).  Every load of the chunk (rows
// clamped to the chunk so no load is conditional) is requested before any
// arithmetic.
template <typename Act, int D, bool OB>
__global__ __launch_bounds__(kNT) void prefill_norm_kernel(PrefillParams p) {
  using io = act_io<Act>;
  constexpr int VPL = 8;           // values per lane
  constexpr int LPR = D / VPL;     // lanes per row
  constexpr int ROWS = kNT / LPR;  // rows per pass
  constexpr int NP = kL / ROWS;    // passes
  static_assert(64 % LPR == 0 && kL % ROWS == 0, "norm split");
  int n, c;
  chunk_of(p, n, c);
  const int h = blockIdx.z;
  const SeqInfo si = seq_info(p, n);
  const int t0 = c * kL;
  if (t0 >= si.len) return;
  const int nc = min(kL, si.len - t0);
  const long long tok0 = si.begin + t0;
  const int tid = threadIdx.x, sub = tid % LPR, rr = tid / LPR;
  const int d0 = sub * VPL;
  // every load of the chunk first, then the padding test: the slot index's
  // round trip overlaps them instead of coming before them (the rows of a
  // padding sequence were never written and are read only to be dropped; the
  // compiler-only fence keeps the loads above the test)
  f32x4 ov[NP][2], zv[NP][2];
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    const int i = min(pass * ROWS + rr, nc - 1);
    const size_t o = ((size_t)(tok0 + i) * p.Hv + h) * D + d0;
    if constexpr (OB) {
      const bf16x8 ob = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.obuf) + o);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int k = 0; k < 4; ++k) ov[pass][hf][k] = static_cast<float>(ob[4 * hf + k]);
    } else {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        ov[pass][hf] = *reinterpret_cast<const f32x4*>(p.obuf + o + 4 * hf);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) zv[pass][hf] = io::load4(p.z, o + 4 * hf);
  }
  f32x4 nw[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) nw[hf] = *reinterpret_cast<const f32x4*>(p.norm_w + d0 + 4 * hf);
  asm volatile("" ::: "memory");
  if (si.slot < 0) {  // padding sequence: zero outputs
    for (int pass = 0; pass < NP; ++pass) {
      const int i = pass * ROWS + rr;
      if (i < nc)
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          const size_t o = ((size_t)(tok0 + i) * p.Hv + h) * D + d0 + k;
          io::store(p.y, o, 0.f);
          if (!OB) p.obuf[o] = 0.f;   // (the bf16 scratch copy is no output)
        }
    }
    return;
  }
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    const int i = pass * ROWS + rr;
    float ss = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int k = 0; k < 4; ++k) ss = fmaf(ov[pass][hf][k], ov[pass][hf][k], ss);
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.0f / sqrtf(ss / D + p.rmseps);
    if (i < nc) {
      const size_t o = ((size_t)(tok0 + i) * p.Hv + h) * D + d0;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 yv;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          yv[k] = nw[hf][k] * ov[pass][hf][k] * inv * silu_fast(zv[pass][hf][k]);
        io::store4(p.y, o + 4 * hf, yv);
      }
    }
  }
}

// ------------------------------------------------------------------ launch

// 16-column blocks per state workgroup: the widest tile (at most 64 columns,
// which fits the registers) that still gives about one workgroup per CU.
// Every tile re-reads the chunk operands of its head, so wider tiles cut that
// traffic; narrower ones spread a few long sequences over more CUs.
static int state_col_blocks(int N, int Hv, int D) {
  int tiles = D > 64 ? D / 64 : 1;
  while (tiles < D / 16 && (long long)N * Hv * tiles < 256) tiles *= 2;
  return D / 16 / tiles;
}

template <typename Act, int D, int K, int NCB>
static void launch_state(const PrefillParams& p, hipStream_t st) {
  // groups of 8 (sequence, K-head) units, each unit r * tiles workgroups
  const long long units = (long long)p.N * p.Hk, per = (long long)p.r * (D / (16 * NCB));
  const long long groups = (units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * per));
  constexpr int nth = state_threads<NCB>();
  if (p.o_bf16)
    prefill_state_kernel<Act, D, K, NCB, true><<<grid, nth, 0, st>>>(p);
  else
    prefill_state_kernel<Act, D, K, NCB, false><<<grid, nth, 0, st>>>(p);
}

template <typename Act, int D, int K>
static hipError_t prefill_run(const PrefillParams& p, int max_chunks, hipStream_t st) {
  // (with no tokens there are no chunks and the scratch may be absent)
  if (!p.inl && p.T > 0) prefill_plan_kernel<<<1, 1024, 0, st>>>(p.cu, p.N, p.T, p.s.chunk_base);
  // per-chunk grid: the real chunks when the prefix travels with the launch
  const dim3 chunks = p.inl ? dim3(p.inl_cb[p.N], 1) : dim3(max_chunks, p.N);
  if (max_chunks > 0) {
    prefill_qk_kernel<Act, D, K><<<dim3(chunks.x, chunks.y, p.Hk), kNT, 0, st>>>(p);
    const long long units = (long long)chunks.x * p.Hk;   // per y
    prefill_wy_kernel<Act, D, K><<<dim3((unsigned)((units + 7) / 8 * 8 * p.r), chunks.y), kNT, 0,
                                   st>>>(p);
  }
  switch (state_col_blocks(p.N, p.Hv, D)) {
    case 1: launch_state<Act, D, K, 1>(p, st); break;
    case 2: launch_state<Act, D, K, 2>(p, st); break;
    case 4: if constexpr (D >= 64) launch_state<Act, D, K, 4>(p, st); break;
    default: return hipErrorInvalidValue;
  }
  if (max_chunks > 0) {
    if (p.o_bf16)
      prefill_norm_kernel<Act, D, true><<<dim3(chunks.x, chunks.y, p.Hv), kNT, 0, st>>>(p);
    else
      prefill_norm_kernel<Act, D, false><<<dim3(chunks.x, chunks.y, p.Hv), kNT, 0, st>>>(p);
  }
  return hipGetLastError();
}

template <typename Act, int D>
static hipError_t prefill_k(const PrefillParams& p, int K, int mc, hipStream_t st) {
  switch (K) {
    case 2: return prefill_run<Act, D, 2>(p, mc, st);
    case 3: return prefill_run<Act, D, 3>(p, mc, st);
    case 4: return prefill_run<Act, D, 4>(p, mc, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename Act>
static hipError_t prefill_d(const PrefillParams& p, int D, int K, int mc, hipStream_t st) {
  switch (D) {
    case 32: return prefill_k<Act, 32>(p, K, mc, st);
    case 64: return prefill_k<Act, 64>(p, K, mc, st);
    case 128: return prefill_k<Act, 128>(p, K, mc, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const gdn_geometry& g, const gdn_layer_weights& w,
                          const gdn_state_pool& pool, const int32_t* cu_seqlens,
                          const int32_t* cu_seqlens_host, int max_len, long long total_tokens,
                          const int32_t* slot_idx, const uint8_t* has_init, int N,
                          const void* qkv_in, const void* z, const void* a,
                          const void* b, void* y, float* o_raw, void* scratch,
                          hipStream_t stream) {
  PrefillParams p;
  p.x = qkv_in;
  p.z = z;
  p.a = a;
  p.b = b;
  p.y = y;
  p.rec = pool.recurrent;
  p.conv = pool.conv;
  p.cu = cu_seqlens;
  p.slot_idx = slot_idx;
  p.has_init = has_init;
  p.conv_w = w.conv_weight;
  p.A_log = w.A_log;
  p.dt_bias = w.dt_bias;
  p.norm_w = w.norm_weight;
  p.s = carve(g, total_tokens, N, scratch);
  p.G = chunk_bound(total_tokens, N);
  p.inl = N <= kInlineSeqs;
  if (p.inl) {
    int run = 0;
    for (int n = 0; n <= N; ++n) {
      p.inl_cu[n] = cu_seqlens_host[n];
      p.inl_cb[n] = run;
      if (n < N) run += (cu_seqlens_host[n + 1] - cu_seqlens_host[n] + kL - 1) / kL;
    }
    // longest first, ties in batch order (insertion sort: at most 64 entries)
    for (int n = 0; n < N; ++n) {
      const int len = cu_seqlens_host[n + 1] - cu_seqlens_host[n];
      int at = n;
      while (at > 0 && cu_seqlens_host[p.inl_order[at - 1] + 1] - cu_seqlens_host[p.inl_order[at - 1]] < len) {
        p.inl_order[at] = p.inl_order[at - 1];
        --at;
      }
      p.inl_order[at] = n;
    }
  }
  p.obuf = o_raw ? o_raw : p.s.o;
  p.o_bf16 = !o_raw && g.act_dtype == GDN_BF16;
  p.T = total_tokens;
  p.N = N;
  p.Hk = g.num_k_heads;
  p.Hv = g.num_v_heads;
  p.C = 2 * g.num_k_heads * g.head_k_dim + g.num_v_heads * g.head_v_dim;
  p.num_slots = pool.num_slots;
  p.r = g.num_v_heads / g.num_k_heads;
  p.l2eps = g.l2norm_eps;
  p.rmseps = g.rmsnorm_eps;
  p.scale = g.scale > 0.f ? g.scale : 1.0f / sqrtf((float)g.head_k_dim);
  const int mc = (max_len + kL - 1) / kL;
  p.max_chunks = mc;
  if (g.act_dtype == GDN_BF16) return prefill_d<__bf16>(p, g.head_k_dim, g.conv_kernel, mc, stream);
  return prefill_d<float>(p, g.head_k_dim, g.conv_kernel, mc, stream);
}

}  // namespace gdn

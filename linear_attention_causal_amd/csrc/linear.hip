// Projections around the layer core: the in_proj_qkv / in_proj_z /
// in_proj_b / in_proj_a input projections and the out_proj output
// projection of the Gated DeltaNet block (cortex commit 95dc874,
// TpQwen3_5GatedDeltaNet bullet: the input projections are split along the
// V-heads, out_proj along its input dimension).  Each is
//     y[m][n] = sum_k x[m][k] w[n][k]
// with bf16 operands, f32 accumulation and a bf16 result; w is row-major
// [N][K] like a Linear layer's weight.  One launch serves up to four
// weights that read the same x (the four input projections of a token).
//
// Two kernels, chosen by the row count M:
//   stream (M <= 32, decode): a weight stream, each weight byte used by at
//     most 32 rows.  A workgroup owns 8, 16 or 32 output columns; its four
//     waves split K and request every weight and input fragment of their K
//     range before the first MFMA, and add their partial tiles through LDS.
//   tile (M > 32): a dense product.  A workgroup owns a BM x BN output tile
//     (128 x 128 with eight waves or 128 x 64 with four, the larger that
//     still gives 128 workgroups, else 64 x 32 with two waves on each half
//     of K, four in all); x and w tiles are
//     staged, one or two 32-wide k-steps per barrier, through three LDS
//     buffers in MFMA fragment order, so each wave reads its operands
//     with linear 16-byte LDS reads, and the input rows are fetched once
//     per BN columns instead of once per 16.  Global loads run six or eight
//     k-steps ahead in registers.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

typedef __bf16 lbf16x8 __attribute__((ext_vector_type(8)));

struct LinParams {
  const __bf16* x;  // [M][ldx]
  int M, K, ldx, count;
  LinearOut out[kMaxLinearOuts];
};

// Weight group of column tile `tile` (uniform across the workgroup).
__device__ __forceinline__ int group_of(const LinParams& p, int tile) {
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxLinearOuts; ++i)
    if (i < p.count && tile >= p.out[i].tile0) g = i;
  return g;
}

__device__ __forceinline__ f32x4 mfma16(lbf16x8 a, lbf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Unconditional 16-byte load of 8 bf16.  Loads are never predicated: a
// branch around a load makes the compiler drain every outstanding load at
// the next use, so callers point a load that is not needed at a valid
// address and zero its value where it is used.
__device__ __forceinline__ lbf16x8 raw8(const __bf16* p) {
  return *reinterpret_cast<const lbf16x8*>(p);
}

__device__ __forceinline__ lbf16x8 keep(lbf16x8 v, bool in) {
  const lbf16x8 zero = {};
  return in ? v : zero;
}

// Store the 16 x 16 tile s (MFMA D layout: D[i][j] at lane j + 16 (i / 4),
// element i % 4) at rows m0.., columns n0.. with bounds guards.
__device__ __forceinline__ void store_tile(const LinearOut& o, int M, int m0, int n0, int lane,
                                           f32x4 s) {
  const int n = n0 + (lane & 15);
  if (n >= o.N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = m0 + 4 * (lane >> 4) + e;
    if (m < M) o.y[(size_t)m * o.ldy + n] = static_cast<__bf16>(s[e]);
  }
}

// CW: the workgroup's output columns when NT == 1 and they are fewer than 16
// (the B operand's upper eight rows then repeat the last column and their
// results are not stored), so that a weight of few columns still spreads
// over every CU.
template <int MT, int NT, int KW, int CW = 16 * NT>
__global__ __launch_bounds__(64 * KW) void linear_stream_kernel(LinParams p) {
  static_assert(CW == 16 * NT || (NT == 1 && CW < 16), "column split");
  constexpr int KB = MT + NT <= 3 ? 16 : 8;  // k-steps requested at once
  __shared__ f32x4 s_part[KW][MT * NT][64];
  const int g = group_of(p, blockIdx.x);
  const LinearOut o = p.out[g];
  const int n0 = ((int)blockIdx.x - o.tile0) * CW, mb = blockIdx.y * 16 * MT;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int li = lane & 15, lk = lane >> 4;
  const int ksteps = (p.K + 31) / 32;
  const int per = (ksteps + KW - 1) / KW;
  const int kb0 = wave * per, kb1 = min(ksteps, kb0 + per);
  // A operand of row tile t: rows mb + 16 t + li of x; B operand of column
  // tile u: row n0 + 16 u + li of w.  Lane li + 16 lk holds k = 32 ks + 8 lk
  // .. +7.  Rows past M or N are clamped to the last one (read, never
  // stored); a k-chunk past K or a step past kb1 reads the row start and
  // counts as zero.
  const __bf16* xr[MT];
  const __bf16* wr[NT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xr[t] = p.x + (size_t)min(mb + 16 * t + li, p.M - 1) * p.ldx;
#pragma unroll
  for (int u = 0; u < NT; ++u) wr[u] = o.w + (size_t)min(n0 + 16 * u + min(li, CW - 1), o.N - 1) * p.K;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = kb0; kb < kb1; kb += KB) {
    lbf16x8 a[KB][MT], b[KB][NT];
    bool in[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int k = 32 * (kb + j) + 8 * lk;
      in[j] = kb + j < kb1 && k < p.K;
      const int off = in[j] ? k : 0;
#pragma unroll
      for (int u = 0; u < NT; ++u) b[j][u] = raw8(wr[u] + off);
#pragma unroll
      for (int t = 0; t < MT; ++t) a[j][t] = raw8(xr[t] + off);
    }
    // keep the whole batch of loads in flight before the first MFMA (the
    // scheduler would otherwise interleave them to save registers)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u)
          acc[t][u] = mfma16(keep(a[j][t], in[j]), b[j][u], acc[t][u]);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) s_part[wave][t * NT + u][lane] = acc[t][u];
  __syncthreads();
  for (int i = wave; i < MT * NT; i += KW) {
    f32x4 s = s_part[0][i][lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) s += s_part[w][i][lane];
    if (CW >= 16 || (lane & 15) < CW)
      store_tile(o, p.M, mb + 16 * (i / NT), n0 + 16 * (i % NT), lane, s);
  }
}

// BM x BN output tile, NW waves as 2 x NW/2, each wave (BM/2) x (2 BN/NW).
// The 128 x 128 tile runs eight waves (two per SIMD, so one wave's LDS and
// barrier waits overlap the other's MFMAs); with four, each wave's registers
// allow only one wave per SIMD.
// K is taken in stages of KS k-steps of 32.  Global loads run DS stages
// ahead of the MFMAs through a ring of DS register stages; each stage is
// copied into one of three LDS buffers two stages before its MFMAs, and its
// fragments are read from LDS one stage before, so LDS latency hides behind
// the previous stage's MFMAs.  One barrier per stage: KS k-steps of MFMAs
// between barriers.
// KG > 1 splits K inside the workgroup: KG groups of NW waves each take a
// contiguous share of the k-steps through their own LDS buffers, in the same
// stages and barriers, and group 0 adds the others' tiles at the end.  A
// small tile then keeps every SIMD of its CU busy.
template <int BM, int BN, int KS, int DS, int NW, int KG = 1>
__global__ __launch_bounds__(64 * NW * KG) void linear_tile_kernel(LinParams p) {
  static_assert(DS >= 3, "the ring holds the two stages ahead of the LDS copy");
  constexpr int NTH = 64 * NW;                      // threads of one k-group
  constexpr int WNW = NW / 2;                       // waves along n (two along m)
  constexpr int TM = BM / 32, TN = BN / (16 * WNW); // 16 x 16 tiles per wave
  constexpr int XP = 4 * BM / NTH, WP = 4 * BN / NTH; // 16-byte pieces per thread per k-step
  static_assert(TN >= 1 && XP >= 1 && WP >= 1, "tile shape");
  // one stage of each operand in fragment order: [k-step][16-row tile][lane] x 16 bytes
  __shared__ lbf16x8 xsg[KG][3][KS][BM / 16][64];
  __shared__ lbf16x8 wsg[KG][3][KS][BN / 16][64];
  const int g = group_of(p, blockIdx.x);
  const LinearOut o = p.out[g];
  const int n0 = ((int)blockIdx.x - o.tile0) * BN, m0 = blockIdx.y * BM;
  const int lane = threadIdx.x & 63, kg = wave_id() / NW, wave = wave_id() - kg * NW;
  const int tid = threadIdx.x - kg * NTH;           // thread within the k-group
  const int wm = wave / WNW, wn = wave % WNW;
  auto& xs = xsg[kg];
  auto& ws = wsg[kg];
  // this group's k-steps: [kg * kspg, (kg + 1) * kspg) of the whole, as a
  // product of depth Kg from column k0 on (every group runs the stages of
  // the largest share; a group past its own skips their MFMAs)
  const int kspg = ((p.K + 31) / 32 + KG - 1) / KG;
  const int k0 = min(p.K, 32 * kspg * kg);
  const int Kg = min(p.K, 32 * kspg * (kg + 1)) - k0;
  const int ksteps = (Kg + 31) / 32;
  const int nst = (ksteps + KS - 1) / KS;           // this group's stages
  const int nall = (kspg + KS - 1) / KS;            // stages every group runs
  const int kb = Kg > 0 ? k0 : 0;   // a group with no k-steps reads row starts only
  // piece q = tid + NTH i: tile row r = q / 4, k-chunk c = q % 4 (the same c
  // for every piece of a thread); its LDS slot is fragment r / 16, lane
  // r % 16 + 16 c.  Rows past M or N are clamped (read, never stored); a
  // k-chunk past K reads the row start, and the MFMAs zero it (a select on
  // loaded data would make the compiler wait for the load where it places
  // the select, which it hoists).
  const int c = tid & 3;
  const __bf16* xsrc[XP];
  const __bf16* wsrc[WP];
  int xslot[XP], wslot[WP];
#pragma unroll
  for (int i = 0; i < XP; ++i) {
    const int r = (tid + NTH * i) >> 2;
    xsrc[i] = p.x + (size_t)min(m0 + r, p.M - 1) * p.ldx + kb;
    xslot[i] = (r >> 4) * 64 + (r & 15) + 16 * c;
  }
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int r = (tid + NTH * i) >> 2;
    wsrc[i] = o.w + (size_t)min(n0 + r, o.N - 1) * p.K + kb;
    wslot[i] = (r >> 4) * 64 + (r & 15) + 16 * c;
  }
  lbf16x8 xr[DS][KS][XP], wr[DS][KS][WP];
  const auto fetch = [&](int st, int S) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k = 32 * (KS * S + kk) + 8 * c;
      const int off = k < Kg ? k : 0;
#pragma unroll
      for (int i = 0; i < XP; ++i) xr[st][kk][i] = raw8(xsrc[i] + off);
#pragma unroll
      for (int i = 0; i < WP; ++i) wr[st][kk][i] = raw8(wsrc[i] + off);
    }
  };
  const auto put = [&](int st, int buf) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int i = 0; i < XP; ++i) (&xs[buf][kk][0][0])[xslot[i]] = xr[st][kk][i];
#pragma unroll
      for (int i = 0; i < WP; ++i) (&ws[buf][kk][0][0])[wslot[i]] = wr[st][kk][i];
    }
  };
  // the last stage, when it holds the end of K inside a k-step or k-steps
  // past K (its lanes past K are zeroed)
  const int last = (Kg == 32 * KS * nst) ? -1 : nst - 1;
  lbf16x8 fa[KS][TM], fb[KS][TN];
  const auto frags = [&](int buf, lbf16x8 (*a)[TM], lbf16x8 (*b)[TN]) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int t = 0; t < TM; ++t) a[kk][t] = xs[buf][kk][wm * TM + t][lane];
#pragma unroll
      for (int u = 0; u < TN; ++u) b[kk][u] = ws[buf][kk][wn * TN + u][lane];
    }
  };
  f32x4 acc[TM][TN];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int u = 0; u < TN; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < DS; ++d) fetch(d, d);
  put(0, 0);
  put(1, 1);
  __syncthreads();
  frags(0, fa, fb);
  // Stage S: read stage S + 1's fragments (LDS buffer (S + 1) % 3), MFMAs of
  // stage S, copy stage S + 2 (ring slot (S + 2) % DS) into buffer (S + 2) %
  // 3, whose fragments were read two barriers ago, and fetch stage S + DS
  // into slot S % DS, copied to LDS two stages ago.  Loads and copies always
  // run (stages past K read row starts); in the guarded form the MFMAs of
  // stages past K are skipped and the lanes past K are zeroed.  The main loop
  // takes only whole groups of DS stages that lie inside K, so it has no
  // branches for the scheduler to stop at.
  const auto step = [&](int d, int S, bool guarded) {
    lbf16x8 na[KS][TM], nb[KS][TN];
    frags((S + 1) % 3, na, nb);
    if (guarded && S == last) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bool in = 32 * (KS * S + kk) + 8 * (lane >> 4) < Kg;
#pragma unroll
        for (int t = 0; t < TM; ++t) fa[kk][t] = keep(fa[kk][t], in);
#pragma unroll
        for (int u = 0; u < TN; ++u) fb[kk][u] = keep(fb[kk][u], in);
      }
    }
    if (!guarded || S < nst) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
          for (int u = 0; u < TN; ++u) acc[t][u] = mfma16(fa[kk][t], fb[kk][u], acc[t][u]);
    }
    put((d + 2) % DS, (S + 2) % 3);
    fetch(d, S + DS);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int t = 0; t < TM; ++t) fa[kk][t] = na[kk][t];
#pragma unroll
      for (int u = 0; u < TN; ++u) fb[kk][u] = nb[kk][u];
    }
  };
  // stages without a K end inside, in every group (the loop bounds are the
  // same for all waves: they meet at every barrier)
  int sfull = nall;
#pragma unroll
  for (int q = 0; q < KG; ++q) {
    const int kq = min(p.K, 32 * kspg * (q + 1)) - min(p.K, 32 * kspg * q);
    const int nq = (kq + 32 * KS - 1) / (32 * KS);
    sfull = min(sfull, kq == 32 * KS * nq ? nq : nq - 1);
  }
  int s0 = 0;
  for (; s0 + DS <= sfull; s0 += DS) {
#pragma unroll
    for (int d = 0; d < DS; ++d) step(d, s0 + d, false);
  }
  for (; s0 < nall; s0 += DS) {
#pragma unroll
    for (int d = 0; d < DS; ++d) step(d, s0 + d, true);
  }
  if constexpr (KG > 1) {
    // the other groups' tiles through LDS (the operand buffers are free
    // after the last barrier), added by group 0
    static_assert(sizeof(xsg) >= (size_t)(KG - 1) * NTH * TM * TN * sizeof(f32x4), "reduce space");
    f32x4* red = reinterpret_cast<f32x4*>(&xsg[0][0][0][0][0]);
    if (kg > 0)
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
          red[(((kg - 1) * NW + wave) * TM * TN + t * TN + u) * 64 + lane] = acc[t][u];
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int q = 1; q < KG; ++q)
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
          acc[t][u] += red[(((q - 1) * NW + wave) * TM * TN + t * TN + u) * 64 + lane];
  }
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int u = 0; u < TN; ++u)
      store_tile(o, p.M, m0 + 16 * (wm * TM + t), n0 + 16 * (wn * TN + u), lane, acc[t][u]);
}

template <typename Kern>
hipError_t launch(Kern kern, LinParams p, const LinearOut* outs, int cols, int rows, int threads,
                  hipStream_t stream) {
  int tiles = 0;
  for (int i = 0; i < kMaxLinearOuts; ++i) {
    p.out[i] = i < p.count ? outs[i] : outs[0];
    p.out[i].tile0 = tiles;
    if (i < p.count) tiles += (outs[i].N + cols - 1) / cols;
  }
  kern<<<dim3(tiles, (p.M + rows - 1) / rows), threads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

LinearPlan linear_plan(int M, const LinearOut* outs, int count) {
  long long cols16 = 0, cols64 = 0, cols128 = 0;
  for (int i = 0; i < count; ++i) {
    cols16 += (outs[i].N + 15) / 16;
    cols64 += (outs[i].N + 63) / 64;
    cols128 += (outs[i].N + 127) / 128;
  }
  if (M <= 32) {
    // two column tiles per workgroup once single tiles would fill the chip
    // (halves the input-row reads per weight byte); for up to 16 rows, half
    // tiles while single ones would not (out_proj of 16 rows at N = 2048:
    // 6.1 -> 5.6 us)
    const int cols = cols16 >= 256 ? 32 : (M <= 16 ? 8 : 16);
    return {LinearPlan::kStream, M <= 16 ? 16 : 32, cols};
  }
  // the largest tile that still gives at least 128 workgroups
  const long long rows128 = (M + 127) / 128;
  if (cols128 * rows128 >= 128) return {LinearPlan::kTile, 128, 128};
  if (cols64 * rows128 >= 128) return {LinearPlan::kTile, 128, 64};
  // otherwise 64 x 32 tiles (two waves on each half of K): twice the
  // workgroups of 64 x 64 tiles, so the product spreads over twice the CUs
  return {LinearPlan::kTile, 64, 32};
}

hipError_t launch_linear(const void* x, int M, int K, int ldx, const LinearOut* outs, int count,
                         hipStream_t stream) {
  LinParams p;
  p.x = static_cast<const __bf16*>(x);
  p.M = M;
  p.K = K;
  p.ldx = ldx;
  p.count = count;
  const LinearPlan plan = linear_plan(M, outs, count);
  if (plan.kind == LinearPlan::kStream) {
    if (plan.rows == 16 && plan.cols == 8)
      return launch(linear_stream_kernel<1, 1, 4, 8>, p, outs, 8, 16, 256, stream);
    if (plan.rows == 16 && plan.cols == 16)
      return launch(linear_stream_kernel<1, 1, 4>, p, outs, 16, 16, 256, stream);
    if (plan.rows == 16) return launch(linear_stream_kernel<1, 2, 4>, p, outs, 32, 16, 256, stream);
    if (plan.cols == 16) return launch(linear_stream_kernel<2, 1, 4>, p, outs, 16, 32, 256, stream);
    return launch(linear_stream_kernel<2, 2, 4>, p, outs, 32, 32, 256, stream);
  }
  if (plan.rows == 128 && plan.cols == 128)
    return launch(linear_tile_kernel<128, 128, 2, 3, 8>, p, outs, 128, 128, 512, stream);
  if (plan.rows == 128)
    return launch(linear_tile_kernel<128, 64, 1, 8, 4>, p, outs, 64, 128, 256, stream);
  return launch(linear_tile_kernel<64, 32, 1, 8, 2, 2>, p, outs, 32, 64, 256, stream);
}

}  // namespace gdn

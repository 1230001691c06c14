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
// At decode row counts this is a weight stream: every weight byte is used
// by at most 16 * MT rows.  One workgroup of four waves per (16-column
// tile, 16*MT-row block); each wave takes a quarter of K, requests its
// weight and input fragments for a batch of k-steps before the first MFMA,
// and the four partial tiles are added through LDS.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

typedef __bf16 lbf16x8 __attribute__((ext_vector_type(8)));

constexpr int kLinNT = 256;  // four waves

struct LinParams {
  const __bf16* x;  // [M][ldx]
  int M, K, ldx, count;
  LinearOut out[kMaxLinearOuts];
};

template <int MT>
__global__ __launch_bounds__(kLinNT) void linear_kernel(LinParams p) {
  constexpr int KB = MT == 1 ? 16 : 8;  // k-steps requested at once per wave
  __shared__ f32x4 s_part[4][MT][64];
  // weight group of this column tile (blockIdx is uniform: scalar selects)
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxLinearOuts; ++i)
    if (i < p.count && (int)blockIdx.x >= p.out[i].tile0) g = i;
  const LinearOut o = p.out[g];
  const int n0 = ((int)blockIdx.x - o.tile0) * 16, mb = blockIdx.y * 16 * MT;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int li = lane & 15, lk = lane >> 4;
  const int ksteps = (p.K + 31) / 32;
  const int per = (ksteps + 3) / 4;
  const int kb0 = wave * per, kb1 = min(ksteps, kb0 + per);
  // A operand of tile t: rows mb + 16 t + li of x; B operand: row n0 + li of w.
  // Lane li + 16 lk holds k = 32 ks + 8 lk .. +7.  Rows past M or N are
  // clamped to the last one (read, never stored); k past K reads as zero.
  const __bf16* xr[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xr[t] = p.x + (size_t)min(mb + 16 * t + li, p.M - 1) * p.ldx + 8 * lk;
  const __bf16* wr = o.w + (size_t)min(n0 + li, o.N - 1) * p.K + 8 * lk;
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const lbf16x8 zero = {};
  for (int kb = kb0; kb < kb1; kb += KB) {
    lbf16x8 a[KB][MT], b[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int ks = min(kb + j, kb1 - 1);  // steps past kb1 are loaded, not used
      const bool in = 32 * ks + 8 * lk < p.K;
      b[j] = in ? *reinterpret_cast<const lbf16x8*>(wr + 32 * ks) : zero;
#pragma unroll
      for (int t = 0; t < MT; ++t)
        a[j][t] = in ? *reinterpret_cast<const lbf16x8*>(xr[t] + 32 * ks) : zero;
    }
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (kb + j < kb1) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j][t], b[j], acc[t], 0, 0, 0);
      }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) s_part[wave][t][lane] = acc[t];
  __syncthreads();
  // wave t sums tile t; D[i][j] sits at lane j + 16 (i / 4), element i % 4
  for (int t = wave; t < MT; t += 4) {
    f32x4 s = s_part[0][t][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) s += s_part[w][t][lane];
    const int n = n0 + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = mb + 16 * t + 4 * lk + e;
      if (m < p.M && n < o.N) o.y[(size_t)m * o.ldy + n] = static_cast<__bf16>(s[e]);
    }
  }
}

}  // namespace

int linear_row_tiles(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

hipError_t launch_linear(const void* x, int M, int K, int ldx, const LinearOut* outs, int count,
                         hipStream_t stream) {
  LinParams p;
  p.x = static_cast<const __bf16*>(x);
  p.M = M;
  p.K = K;
  p.ldx = ldx;
  p.count = count;
  int tiles = 0;
  for (int i = 0; i < kMaxLinearOuts; ++i) {
    p.out[i] = i < count ? outs[i] : outs[0];
    p.out[i].tile0 = tiles;
    if (i < count) tiles += (outs[i].N + 15) / 16;
  }
  const int mt = linear_row_tiles(M);
  const dim3 grid(tiles, (M + 16 * mt - 1) / (16 * mt));
  switch (mt) {
    case 1: linear_kernel<1><<<grid, kLinNT, 0, stream>>>(p); break;
    case 2: linear_kernel<2><<<grid, kLinNT, 0, stream>>>(p); break;
    default: linear_kernel<4><<<grid, kLinNT, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace gdn

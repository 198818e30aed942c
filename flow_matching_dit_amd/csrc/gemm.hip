// GEMMs of the action head for gfx950.
//
//  * gemm_mfma_kernel: bf16 activations x (bf16 | e4m3) weights on the matrix cores
//    (v_mfma_f32_16x16x32_bf16), fp32 accumulation. Tiles of A [BM x 64] and
//    W [BN x 64] are staged through LDS, double buffered, with the next tile's
//    global loads issued before the current tile's MFMAs. e4m3 weights are decoded
//    to bf16 (exactly) on their way into LDS; the per-column scale is applied in the
//    epilogue. Serves the DiT projections, the VL key/value projection and the
//    per-embodiment linears of width D.
//  * gemm_valu_kernel: fp32 FMA on the vector ALUs for any (A, W) storage types.
//    Serves the fp32 path, the input-independent tables and the per-embodiment
//    linears whose K or N is the small action/state width.
//
// Both read a group/category description (GemmArgs) so one launch covers the
// per-sample weight gather of the per-embodiment linear (the batched product over
// W[ids] on the architecture page, "Embodiment-specific projectors"), and finish
// with a fused epilogue (bias, activation, residual add, head-major scatter, Euler).
#include "kcommon.h"
#include "kernels.h"

namespace gr00t {

__device__ __forceinline__ float apply_act(int act, float v) {
  switch (act) {
    case ACT_RELU: return fmaxf(v, 0.0f);
    case ACT_SILU: return silu_f(v);
    case ACT_GELU: return gelu_erf(v);
    default: return v;
  }
}

__device__ __forceinline__ void epi_apply(const Epi& e, int g, int r, int n, float v, int cat) {
  if (e.add_tab) v += e.add_tab[(long)cat * e.add_cstride + n];
  v = apply_act(e.act, v);
  const long row = (long)g * e.out_gstride + e.out_row_off + r;
  switch (e.kind) {
    case EPI_STORE: {
      const long idx = row * e.out_ld + n;
      if (e.out_f32) ((float*)e.out)[idx] = v;
      else st((bf16*)e.out + idx, v);
    } break;
    case EPI_RESID_ADD: {
      float* p = (float*)e.out + row * e.out_ld + n;
      *p = *p + v;
    } break;
    case EPI_EULER: {
      float* p = (float*)e.out + row * e.out_ld + n;
      *p = *p + e.dt * v;
    } break;
    case EPI_HEADS: {
      const int sec = n / e.width;
      const int which = sec % e.nwhich;
      const int layer = sec / e.nwhich;
      const int c = n - sec * e.width;
      const int head = c / e.hd;
      const int d = c - head * e.hd;
      const int b = (int)(row / e.pos_per_b);
      const int pos = (int)(row - (long)b * e.pos_per_b);
      const long idx = (long)layer * e.layer_stride +
                       (((long)b * e.nh + head) * e.pos_per_b + pos) * e.hd + d;
      if (e.out_f32) ((float*)e.heads[which])[idx] = v;
      else st((bf16*)e.heads[which] + idx, v);
    } break;
  }
}

// ------------------------------------------------------------------------------------
// Vector-ALU GEMM: 64 x 64 tile, 256 threads, 4 x 4 outputs per thread.
// ------------------------------------------------------------------------------------
template <typename TA, typename TW>
__global__ __launch_bounds__(256) void gemm_valu_kernel(GemmArgs a, Epi e) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Ws[BK][BN + 4];
  const int g = blockIdx.z;
  const int cat = a.ids ? a.ids[g] : 0;
  const int r0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const TA* A = (const TA*)a.A + ((long)g * a.a_gstride + a.a_row_off) * a.lda;
  const TW* W = (const TW*)a.W + (long)cat * a.w_cstride;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  const int lr = t / 4, lk = (t % 4) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < a.K; k0 += BK) {
    const int r = r0 + lr, n = n0 + lr;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = k0 + lk + q;
      As[lk + q][lr] = (r < a.rows && k < a.K) ? ld(A + (long)r * a.lda + k) : 0.0f;
      Ws[lk + q][lr] = (n < a.N && k < a.K) ? ld(W + (long)n * a.K + k) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = Ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty * 4 + i;
    if (r >= a.rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= a.N) continue;
      float v = acc[i][j];
      if (a.wscale) v *= a.wscale[(long)cat * a.s_cstride + n];
      if (a.bias) v += a.bias[(long)cat * a.b_cstride + n];
      epi_apply(e, g, r, n, v, cat);
    }
  }
}

// ------------------------------------------------------------------------------------
// MFMA GEMM. Block tile BM x BN, BK = 64, waves arranged WM x WN, each wave owning a
// (BM/WM) x (BN/WN) sub-tile made of 16 x 16 MFMA fragments.
//
// v_mfma_f32_16x16x32_bf16 operand layout (wave64): A fragment (16 rows x 32 k): lane l
// holds row l%16, k = 8*(l/16) .. +7; B fragment (32 k x 16 cols): lane l holds column
// l%16, the same k range; the 16 x 16 fp32 result: lane l holds column l%16, rows
// 4*(l/16) .. +3.
// ------------------------------------------------------------------------------------
constexpr int MF_BK = 64;
constexpr int MF_LDS_LD = MF_BK + 8;  // bf16 elements per LDS row (16 B pad: conflict-free b128 reads)

template <int BM, int BN, int WM, int WN, bool FP8>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_kernel(GemmArgs a, Epi e) {
  constexpr int NT = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold at least one 16x16 fragment");
  constexpr int A_CHUNKS = BM * 8;                      // 16-byte chunks of bf16
  constexpr int B_CHUNKS = FP8 ? BN * 4 : BN * 8;       // 16-byte chunks of W
  constexpr int A_PER = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER = (B_CHUNKS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * MF_LDS_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * MF_LDS_LD];

  const int g = blockIdx.z;
  const int cat = a.ids ? a.ids[g] : 0;
  const int r0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const uint16_t* A = (const uint16_t*)a.A + ((long)g * a.a_gstride + a.a_row_off) * a.lda;
  const uint8_t* W8 = (const uint8_t*)a.W + (long)cat * a.w_cstride;          // FP8
  const uint16_t* W16 = (const uint16_t*)a.W + (long)cat * a.w_cstride;       // bf16
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave / WN, wn = wave % WN;

  uint4 ra[A_PER], rb[B_PER];

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = t + i * NT;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < A_CHUNKS) {
        const int row = c >> 3, kc = (c & 7) * 8;
        const int gr = r0 + row;
        if (gr < a.rows && k0 + kc < a.K) v = *(const uint4*)(A + (long)gr * a.lda + k0 + kc);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = t + i * NT;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < B_CHUNKS) {
        if (FP8) {
          const int n = c >> 2, kc = (c & 3) * 16;
          const int gn = n0 + n;
          if (gn < a.N && k0 + kc < a.K) v = *(const uint4*)(W8 + (long)gn * a.K + k0 + kc);
        } else {
          const int n = c >> 3, kc = (c & 7) * 8;
          const int gn = n0 + n;
          if (gn < a.N && k0 + kc < a.K) v = *(const uint4*)(W16 + (long)gn * a.K + k0 + kc);
        }
      }
      rb[i] = v;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = t + i * NT;
      if (c < A_CHUNKS) {
        const int row = c >> 3, kc = (c & 7) * 8;
        *(uint4*)&As[buf][row * MF_LDS_LD + kc] = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = t + i * NT;
      if (c < B_CHUNKS) {
        if (FP8) {
          const int n = c >> 2, kc = (c & 3) * 16;
          const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
          uint32_t o[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[2 * q] = (uint32_t)e4m3_to_bf16(w[q] & 0xFF) | ((uint32_t)e4m3_to_bf16((w[q] >> 8) & 0xFF) << 16);
            o[2 * q + 1] =
                (uint32_t)e4m3_to_bf16((w[q] >> 16) & 0xFF) | ((uint32_t)e4m3_to_bf16(w[q] >> 24) << 16);
          }
          *(uint4*)&Bs[buf][n * MF_LDS_LD + kc] = make_uint4(o[0], o[1], o[2], o[3]);
          *(uint4*)&Bs[buf][n * MF_LDS_LD + kc + 8] = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
          const int n = c >> 3, kc = (c & 7) * 8;
          *(uint4*)&Bs[buf][n * MF_LDS_LD + kc] = rb[i];
        }
      }
    }
  };

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (a.K + MF_BK - 1) / MF_BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * MF_BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[FM], bfr[FN];
      const int koff = ks * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *(const bf16x8_t*)&As[buf][(wm * TM + i * 16 + (lane & 15)) * MF_LDS_LD + koff];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *(const bf16x8_t*)&Bs[buf][(wn * TN + j * 16 + (lane & 15)) * MF_LDS_LD + koff];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * TN + j * 16 + (lane & 15);
    if (n >= a.N) continue;
    const float sc = a.wscale ? a.wscale[(long)cat * a.s_cstride + n] : 1.0f;
    const float bi = a.bias ? a.bias[(long)cat * a.b_cstride + n] : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + wm * TM + i * 16 + (lane >> 4) * 4 + q;
        if (r < a.rows) epi_apply(e, g, r, n, acc[i][j][q] * sc + bi, cat);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------
template <typename TA, typename TW>
static hipError_t valu_go(const GemmArgs& a, const Epi& e, hipStream_t s) {
  dim3 grid((a.N + 63) / 64, (a.rows + 63) / 64, a.groups);
  hipLaunchKernelGGL((gemm_valu_kernel<TA, TW>), grid, dim3(256), 0, s, a, e);
  return hipGetLastError();
}

hipError_t launch_gemm_valu(const GemmArgs& a, const Epi& e, DType at, DType wt, hipStream_t s) {
  if (a.rows <= 0 || a.N <= 0 || a.groups <= 0) return hipSuccess;
  if (at == DT_F32 && wt == DT_F32) return valu_go<float, float>(a, e, s);
  if (at == DT_F32 && wt == DT_BF16) return valu_go<float, bf16>(a, e, s);
  if (at == DT_BF16 && wt == DT_BF16) return valu_go<bf16, bf16>(a, e, s);
  if (at == DT_BF16 && wt == DT_F32) return valu_go<bf16, float>(a, e, s);
  if (at == DT_F32 && wt == DT_FP8) return valu_go<float, fp8e4m3>(a, e, s);
  if (at == DT_BF16 && wt == DT_FP8) return valu_go<bf16, fp8e4m3>(a, e, s);
  return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN>
static hipError_t mfma_go(const GemmArgs& a, const Epi& e, bool fp8, hipStream_t s) {
  dim3 grid((a.N + BN - 1) / BN, (a.rows + BM - 1) / BM, a.groups);
  if (fp8)
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, true>), grid, dim3(64 * WM * WN), 0, s, a, e);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, false>), grid, dim3(64 * WM * WN), 0, s, a, e);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmArgs& a, const Epi& e, DType wt, hipStream_t s) {
  if (a.rows <= 0 || a.N <= 0 || a.groups <= 0) return hipSuccess;
  if ((a.K % 8) != 0 || (a.lda % 8) != 0) return hipErrorInvalidValue;
  const bool fp8 = (wt == DT_FP8);
  if (!fp8 && wt != DT_BF16) return hipErrorInvalidValue;
  if (fp8 && (a.K % 16) != 0) return hipErrorInvalidValue;
  const long tiles128 = (long)((a.N + 127) / 128) * ((a.rows + 127) / 128) * a.groups;
  if (a.rows <= 16) return mfma_go<16, 64, 1, 4>(a, e, fp8, s);
  if (a.rows <= 32) return mfma_go<32, 64, 1, 4>(a, e, fp8, s);
  if (a.rows <= 64 || tiles128 < 256) return mfma_go<64, 128, 2, 2>(a, e, fp8, s);
  return mfma_go<128, 128, 2, 2>(a, e, fp8, s);
}

}  // namespace gr00t

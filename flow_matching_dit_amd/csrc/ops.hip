// Non-GEMM kernels of the action head for gfx950: LayerNorm / adaptive LayerNorm,
// masked multi-head attention, and the small per-call kernels (masks, ids, noise,
// output, timestep sinusoids).
#include <math.h>

#include "kcommon.h"
#include "kernels.h"

namespace gr00t {

// ------------------------------------------------------------------------------------
// LayerNorm, one wave64 per row (row statistics by wave reductions). Covers the
// vision-language LayerNorm (gain and bias), the timestep-conditioned adaLN
// LN(h) * (1 + scale) + shift of every block and of the output, and the plain norm3
// ("Model architecture", "Transformer block structure").
// ------------------------------------------------------------------------------------
template <typename TX, typename TY>
__global__ __launch_bounds__(256) void layernorm_kernel(const TX* __restrict__ x, long ldx, TY* __restrict__ y,
                                                        long ldy, int rows, int D, const float* __restrict__ gamma,
                                                        const float* __restrict__ beta,
                                                        const float* __restrict__ ada,
                                                        const int* __restrict__ row_idx,
                                                        const int* __restrict__ row_count) {
  constexpr int MAXPER = 32;  // D <= 2048
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  if (row_count && row >= *row_count) return;
  const TX* xr = x + (long)(row_idx ? row_idx[row] : row) * ldx;
  float v[MAXPER];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    const int c = lane + i * 64;
    v[i] = (c < D) ? ld(xr + c) : 0.0f;
    s += v[i];
  }
  const float mean = wave_sum(s) / (float)D;
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    const int c = lane + i * 64;
    const float d = v[i] - mean;
    s2 += (c < D) ? d * d : 0.0f;
  }
  const float var = wave_sum(s2) / (float)D;
  const float rstd = 1.0f / sqrtf(var + 1e-5f);
  TY* yr = y + (long)row * ldy;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    const int c = lane + i * 64;
    if (c < D) {
      float o = (v[i] - mean) * rstd;
      if (gamma) o = o * gamma[c] + beta[c];
      if (ada) o = o * (1.0f + ada[c]) + ada[D + c];
      st(yr + c, o);
    }
  }
}

hipError_t launch_layernorm(const void* x, DType xt, long ldx, void* y, DType yt, long ldy, int rows, int D,
                            const float* gamma, const float* beta, const float* ada, hipStream_t s, const int* row_idx,
                            const int* row_count) {
  if (rows <= 0) return hipSuccess;
  if (D > 2048) return hipErrorInvalidValue;
  dim3 grid((rows + 3) / 4);
  if (xt == DT_F32 && yt == DT_F32)
    hipLaunchKernelGGL((layernorm_kernel<float, float>), grid, dim3(256), 0, s, (const float*)x, ldx, (float*)y, ldy,
                       rows, D, gamma, beta, ada, row_idx, row_count);
  else if (xt == DT_F32 && yt == DT_BF16)
    hipLaunchKernelGGL((layernorm_kernel<float, bf16>), grid, dim3(256), 0, s, (const float*)x, ldx, (bf16*)y, ldy,
                       rows, D, gamma, beta, ada, row_idx, row_count);
  else if (xt == DT_BF16 && yt == DT_BF16)
    hipLaunchKernelGGL((layernorm_kernel<bf16, bf16>), grid, dim3(256), 0, s, (const bf16*)x, ldx, (bf16*)y, ldy,
                       rows, D, gamma, beta, ada, row_idx, row_count);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Residual add of split-K partial sums fused with the next (ada)LayerNorm: one wave per
// row, float4 accesses (lane owns columns 4*lane + 256*i .. +3); the row of h is updated
// in place (h + p_0 + p_1 + ..., fixed order) and normalised. D % 4 == 0, D <= 2048.
// TY = uint8_t (W8A8): the normalised row is rounded to bf16 as for a bf16 output, then
// written as the e4m3 codes of quant_rows_kernel (row scale amax / 448 into qscale[row],
// codes of the correctly rounded quotients), so the GEMM reads it without a separate pass.
template <typename TY, int NS>
__global__ __launch_bounds__(256) void resid_layernorm_kernel(float* __restrict__ h, const float* __restrict__ part,
                                                              long split_stride, TY* __restrict__ y, int rows, int D,
                                                              const float* __restrict__ ada_base, int ada_rows,
                                                              long ada_stride, float* __restrict__ qscale) {
  constexpr bool Q8 = sizeof(TY) == 1;
  constexpr int MAXV = 8;  // float4 per lane: 8 * 4 * 64 = 2048 columns
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* ada = ada_base ? ada_base + (ada_rows > 0 ? (long)(row / ada_rows) * ada_stride : 0) : nullptr;
  float* hr = h + (long)row * D;
  float4 v[MAXV];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = 4 * lane + 256 * i;
    float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (c < D) {
      x = *(const float4*)(hr + c);
#pragma unroll
      for (int p = 0; p < NS; ++p) {
        const float4 q = *(const float4*)(part + (long)p * split_stride + (long)row * D + c);
        x.x += q.x;
        x.y += q.y;
        x.z += q.z;
        x.w += q.w;
      }
      if (NS > 0) *(float4*)(hr + c) = x;
    }
    v[i] = x;
    s += (x.x + x.y) + (x.z + x.w);
  }
  const float mean = wave_sum(s) / (float)D;
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = 4 * lane + 256 * i;
    if (c < D) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      s2 += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / (float)D + 1e-5f);
  TY* yr = y + (long)row * D;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = 4 * lane + 256 * i;
    if (c < D) {
      float o[4] = {(v[i].x - mean) * rstd, (v[i].y - mean) * rstd, (v[i].z - mean) * rstd, (v[i].w - mean) * rstd};
      if (ada) {
        const float4 sc = *(const float4*)(ada + c);
        const float4 sh = *(const float4*)(ada + D + c);
        o[0] = o[0] * (1.0f + sc.x) + sh.x;
        o[1] = o[1] * (1.0f + sc.y) + sh.y;
        o[2] = o[2] * (1.0f + sc.z) + sh.z;
        o[3] = o[3] * (1.0f + sc.w) + sh.w;
      }
      if constexpr (Q8) {
        const uint32_t b01 = bf16x2_bits(o[0], o[1]), b23 = bf16x2_bits(o[2], o[3]);
        v[i] = make_float4(bf16_to_f(b01 & 0xFFFFu), bf16_to_f(b01 >> 16), bf16_to_f(b23 & 0xFFFFu),
                           bf16_to_f(b23 >> 16));
      } else if (sizeof(TY) == 4) {
        *(float4*)((float*)yr + c) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        *(uint2*)((uint16_t*)yr + c) = make_uint2(bf16x2_bits(o[0], o[1]),
                                                  bf16x2_bits(o[2], o[3]));
      }
    }
  }
  if constexpr (Q8) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (4 * lane + 256 * i < D)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    amax = wave_max(amax);
    const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (lane == 0) qscale[row] = sc;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = 4 * lane + 256 * i;
      if (c < D) {
        int q = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(v[i].x, sc), __fdiv_rn(v[i].y, sc), 0, false);
        q = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(v[i].z, sc), __fdiv_rn(v[i].w, sc), q, true);
        *(uint32_t*)((uint8_t*)yr + c) = (uint32_t)q;
      }
    }
  }
}

// The same for bf16 / fp32 outputs with one workgroup of NW waves per row: thread t owns
// columns 2 t + 128 NW i .. +1, so NW waves share a row and NW times as many loads are in
// flight as with a wave per row (at B = 64 the 1088 rows give about one wave per SIMD). The
// row's sums are wave sums added in wave order through LDS.
template <typename TY, int NS, int NW>
__global__ __launch_bounds__(64 * NW) void resid_layernorm_row_kernel(float* __restrict__ h, const float* __restrict__ part,
                                                                      long split_stride, TY* __restrict__ y, int D,
                                                                      const float* __restrict__ ada_base, int ada_rows,
                                                                      long ada_stride) {
  constexpr int NTR = 64 * NW, MAXV = (2048 + 2 * NTR - 1) / (2 * NTR);  // float2 per thread, up to 2048 columns
  __shared__ float red[2][NW];
  const int row = blockIdx.x;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const float* ada = ada_base ? ada_base + (ada_rows > 0 ? (long)(row / ada_rows) * ada_stride : 0) : nullptr;
  float* hr = h + (long)row * D;
  float2 v[MAXV];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = 2 * t + 2 * NTR * i;
    float2 x = make_float2(0.0f, 0.0f);
    if (c < D) {
      x = *(const float2*)(hr + c);
#pragma unroll
      for (int p = 0; p < NS; ++p) {
        const float2 q = *(const float2*)(part + (long)p * split_stride + (long)row * D + c);
        x.x += q.x;
        x.y += q.y;
      }
      if (NS > 0) *(float2*)(hr + c) = x;
    }
    v[i] = x;
    s += x.x + x.y;
  }
  s = wave_sum(s);
  if (lane == 0) red[0][wave] = s;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += red[0][w];
  const float mean = tot / (float)D;
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if (2 * t + 2 * NTR * i < D) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean;
      s2 += a0 * a0 + a1 * a1;
    }
  }
  s2 = wave_sum(s2);
  if (lane == 0) red[1][wave] = s2;
  __syncthreads();
  float tot2 = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot2 += red[1][w];
  const float rstd = 1.0f / sqrtf(tot2 / (float)D + 1e-5f);
  TY* yr = y + (long)row * D;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = 2 * t + 2 * NTR * i;
    if (c < D) {
      float o0 = (v[i].x - mean) * rstd, o1 = (v[i].y - mean) * rstd;
      if (ada) {
        const float2 sc = *(const float2*)(ada + c);
        const float2 sh = *(const float2*)(ada + D + c);
        o0 = o0 * (1.0f + sc.x) + sh.x;
        o1 = o1 * (1.0f + sc.y) + sh.y;
      }
      if (sizeof(TY) == 4) *(float2*)((float*)yr + c) = make_float2(o0, o1);
      else *(uint32_t*)((uint16_t*)yr + c) = bf16x2_bits(o0, o1);
    }
  }
}

constexpr int RLN_FEW_ROWS = 256;
template <typename TY>
static hipError_t resid_ln_go(float* h, const float* partials, int nsplit, long split_stride, TY* y, int rows, int D,
                              const float* ada, int ada_rows, long ada_stride, float* qscale, hipStream_t s) {
  if (sizeof(TY) != 1) {  // bf16 / fp32 outputs: a workgroup per row (8 waves when there are few rows)
#define GR00T_RLN_CASE(N)                                                                                       \
  case N:                                                                                                       \
    if (rows < RLN_FEW_ROWS)                                                                                    \
      hipLaunchKernelGGL((resid_layernorm_row_kernel<TY, N, 8>), dim3(rows), dim3(512), 0, s, h, partials,      \
                         split_stride, y, D, ada, ada_rows, ada_stride);                                        \
    else                                                                                                        \
      hipLaunchKernelGGL((resid_layernorm_row_kernel<TY, N, 4>), dim3(rows), dim3(256), 0, s, h, partials,      \
                         split_stride, y, D, ada, ada_rows, ada_stride);                                        \
    break;
    switch (nsplit) {
      GR00T_RLN_CASE(0)
      GR00T_RLN_CASE(1)
      GR00T_RLN_CASE(2)
      GR00T_RLN_CASE(3)
      GR00T_RLN_CASE(4)
      GR00T_RLN_CASE(5)
      GR00T_RLN_CASE(6)
      GR00T_RLN_CASE(7)
      GR00T_RLN_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef GR00T_RLN_CASE
    return hipGetLastError();
  }
  dim3 grid((rows + 3) / 4), blk(256);
  switch (nsplit) {
    case 0: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 0>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 1: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 1>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 2: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 2>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 3: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 3>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 4: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 4>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 5: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 5>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 6: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 6>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 7: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 7>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    case 8: hipLaunchKernelGGL((resid_layernorm_kernel<TY, 8>), grid, blk, 0, s, h, partials, split_stride, y, rows, D, ada, ada_rows, ada_stride, qscale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resid_layernorm(float* h, const float* partials, int nsplit, long split_stride, void* y, DType yt,
                                  int rows, int D, const float* ada, hipStream_t s, int ada_rows, long ada_stride,
                                  float* qscale) {
  if (rows <= 0) return hipSuccess;
  if (D > 2048 || (D % 4) != 0 || ada_rows < 0) return hipErrorInvalidValue;
  if (!partials) nsplit = 0;
  if (yt == DT_F32)
    return resid_ln_go<float>(h, partials, nsplit, split_stride, (float*)y, rows, D, ada, ada_rows, ada_stride, nullptr,
                              s);
  if (yt == DT_BF16)
    return resid_ln_go<bf16>(h, partials, nsplit, split_stride, (bf16*)y, rows, D, ada, ada_rows, ada_stride, nullptr,
                             s);
  if (yt == DT_FP8 && qscale)
    return resid_ln_go<uint8_t>(h, partials, nsplit, split_stride, (uint8_t*)y, rows, D, ada, ada_rows, ada_stride,
                                qscale, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------
// Attention on the vector ALUs (fp32 path): one workgroup per (head, sample); keys
// streamed in chunks of 64 through LDS with an online (running max / running sum)
// softmax in fp32. Self-attention blocks pass the S state+action tokens as keys;
// cross-attention blocks pass the cached VL keys/values with the block's key mask
// ("AlternateVLDiT variant").
// ------------------------------------------------------------------------------------
constexpr int AT_KC = 64;
constexpr int AT_SMAX = 65;
constexpr int AT_HDMAX = 64;
constexpr int AT_OPT = (AT_SMAX * AT_HDMAX + 255) / 256;  // outputs owned per thread

template <typename T>
__global__ __launch_bounds__(256) void attention_valu_kernel(AttnArgs a) {
  __shared__ float Qs[AT_SMAX][AT_HDMAX + 1];
  __shared__ float Ks[AT_KC][AT_HDMAX + 1];
  __shared__ float Vs[AT_KC][AT_HDMAX + 1];
  __shared__ float Ps[AT_SMAX][AT_KC + 1];
  __shared__ float m_s[AT_SMAX], l_s[AT_SMAX], al_s[AT_SMAX];
  __shared__ int adm[AT_KC];

  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int S = a.S, hd = a.hd, Lk = a.Lk, Lp = a.Lp, nh = a.nh;
  const T* q = (const T*)a.q + (long)(b * nh + h) * S * hd;
  const T* k = (const T*)a.k + (long)(b * nh + h) * Lp * hd;
  const T* vt = (const T*)a.vt + (long)(b * nh + h) * hd * Lp;
  const float scale = 1.0f / sqrtf((float)hd);

  for (int i = t; i < S * hd; i += 256) Qs[i / hd][i % hd] = ld(q + i) * scale;
  for (int i = t; i < S; i += 256) {
    m_s[i] = -INFINITY;
    l_s[i] = 0.0f;
  }
  float oacc[AT_OPT];
#pragma unroll
  for (int j = 0; j < AT_OPT; ++j) oacc[j] = 0.0f;

  for (int j0 = 0; j0 < Lk; j0 += AT_KC) {
    const int nk = min(AT_KC, Lk - j0);
    __syncthreads();
    for (int i = t; i < AT_KC * hd; i += 256) {
      const int jj = i / hd, d = i - jj * hd;
      const bool in = jj < nk;
      Ks[jj][d] = in ? ld(k + (long)(j0 + jj) * hd + d) : 0.0f;
    }
    for (int i = t; i < AT_KC * hd; i += 256) {
      const int d = i / AT_KC, jj = i - d * AT_KC;
      const int pos = j0 + jj;  // values cached [pos / 32][hd][pos % 32]
      Vs[jj][d] = (jj < nk) ? ld(vt + (long)(pos >> 5) * hd * 32 + d * 32 + (pos & 31)) : 0.0f;
    }
    if (t < AT_KC) adm[t] = (t < nk) && (a.mask == nullptr || (a.mask[(long)b * Lk + j0 + t] & a.mask_bit));
    __syncthreads();
    for (int i = t; i < S * AT_KC; i += 256) {
      const int s = i / AT_KC, jj = i - s * AT_KC;
      float sc = -INFINITY;
      if (adm[jj]) {
        float acc = 0.0f;
        for (int d = 0; d < hd; ++d) acc = fmaf(Qs[s][d], Ks[jj][d], acc);
        sc = acc;
      }
      Ps[s][jj] = sc;
    }
    __syncthreads();
    for (int s = wave; s < S; s += 4) {
      const float sc = Ps[s][lane];
      const float mx = wave_max(sc);
      const float mold = m_s[s];
      const float mnew = fmaxf(mold, mx);
      const float p = (sc == -INFINITY) ? 0.0f : expf(sc - mnew);
      const float alpha = (mnew == -INFINITY) ? 1.0f : expf(mold - mnew);
      const float ps = wave_sum(p);
      Ps[s][lane] = p;
      if (lane == 0) {
        l_s[s] = l_s[s] * alpha + ps;
        m_s[s] = mnew;
        al_s[s] = alpha;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < AT_OPT; ++j) {
      const int p = t + j * 256;
      if (p < S * hd) {
        const int s = p / hd, d = p - s * hd;
        float acc = oacc[j] * al_s[s];
        for (int jj = 0; jj < nk; ++jj) acc = fmaf(Ps[s][jj], Vs[jj][d], acc);
        oacc[j] = acc;
      }
    }
  }
  __syncthreads();
  T* o = (T*)a.o;
#pragma unroll
  for (int j = 0; j < AT_OPT; ++j) {
    const int p = t + j * 256;
    if (p < S * hd) {
      const int s = p / hd, d = p - s * hd;
      const float l = l_s[s];
      st(o + ((long)(b * S + s) * nh + h) * hd + d, l > 0.0f ? oacc[j] / l : 0.0f);
    }
  }
}

// ------------------------------------------------------------------------------------
// Attention on the matrix cores (bf16). For a 32-key tile, S^T = K Q^T is formed per
// 16-query fragment with v_mfma_f32_16x16x32_bf16, so each lane holds the scores of
// one query against 8 keys; the tile's keys are enumerated so that those 8 keys are
// contiguous, which makes the exponentiated scores directly the B operand of
// O^T += V^T P^T (values cached transposed per 32-key tile, [L/32][hd][32]). Running max / sum in fp32 with
// exp2; tiles with no admitted key are not multiplied.
//  * attention_mfma_kernel: one workgroup (4 or 8 waves) per (head, sample); wave w
//    takes the tiles w, w+NW, ...; the waves' partial results are merged through LDS.
//    For few (sample, head) pairs (small batches).
//  * attention_wave_kernel: one wave per (sample, head) streaming all its tiles; for
//    many pairs.
// ------------------------------------------------------------------------------------
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));


// K fragments of the two 16-key halves of key tile kt (row r of half th is key
// 8*(r/4) + 4*th + r%4, so lane group g ends with the scores of keys 8g .. 8g+7) and the
// V^T fragments (head dim hf*16 + c16, keys 8g .. +7 of the tile). Rows of the tile past Lk hold
// finite values (the caller's padding contract) and get weight 0.
template <int HD>
__device__ __forceinline__ void attn_load_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int Lp, int kt, int g,
                                               int c16, bf16x8_v (&kf)[2][(HD + 31) / 32], bf16x8_v (&vf)[HD / 16]) {
  constexpr int KS = (HD + 31) / 32, HF = HD / 16;
  const int base = kt * 32;
#pragma unroll
  for (int th = 0; th < 2; ++th) {
    const int key = base + 8 * (c16 >> 2) + 4 * th + (c16 & 3);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 32 + g * 8;  // head dims past HD read 0 (zero padding of the last k step)
      kf[th][ks] = __builtin_bit_cast(bf16x8_v, buf_load16(kr, d0 < HD ? (key * HD + d0) * 2 : OOB));
    }
  }
  // values cached [tile][hd][32]: the 16 head-dim rows of a fragment are 1 KB of contiguous memory
#pragma unroll
  for (int hf = 0; hf < HF; ++hf)
    vf[hf] = __builtin_bit_cast(bf16x8_v, buf_load16(vr, ((kt * HD + hf * 16 + c16) * 32 + 8 * g) * 2));
}

// One key tile of the online softmax: scores S^T = K Q^T on the matrix cores, running
// max m (in units of log2 e / sqrt(hd), folded into sl2) and sum l per query, O^T += V^T P^T.
// mybits: admitted-key bits of keys 8g .. 8g+7 of the tile; full: every key of the tile is
// admitted (wave-uniform), so no key needs masking. The max is taken on the raw scores
// (sl2 > 0) and each probability is exp2(score * sl2 - m) with one fma.
template <int HD, int QF>
__device__ __forceinline__ void attn_tile(const bf16x8_v (&qfr)[QF][(HD + 31) / 32], floatx4_t (&acc)[QF][HD / 16],
                                          float (&m)[QF], float (&l)[QF], const bf16x8_v (&kf)[2][(HD + 31) / 32],
                                          const bf16x8_v (&vf)[HD / 16], uint32_t mybits, bool full, float sl2) {
  constexpr int KS = (HD + 31) / 32, HF = HD / 16;
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    floatx4_t sc[2];
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      floatx4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[th][ks], qfr[qf][ks], z, 0, 0, 0);
      sc[th] = z;
    }
    float tmax = -INFINITY;
    if (full) {
#pragma unroll
      for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, sc[i >> 2][i & 3]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) tmax = fmaxf(tmax, ((mybits >> i) & 1u) ? sc[i >> 2][i & 3] : -INFINITY);
    }
    tmax = across_rows_16_32(tmax, MaxOp{});
    const float mnew = fmaxf(m[qf], tmax * sl2);
    const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m[qf] - mnew);
    float p[8];
    if (full) {
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sc[i >> 2][i & 3], sl2, -mnew));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        p[i] = ((mybits >> i) & 1u) ? __builtin_amdgcn_exp2f(fmaf(sc[i >> 2][i & 3], sl2, -mnew)) : 0.0f;
    }
    float psum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    psum = across_rows_16_32(psum, SumOp{});
    l[qf] = l[qf] * alpha + psum;
    m[qf] = mnew;
    const bf16x8_v pf = __builtin_bit_cast(
        bf16x8_v, make_uint4(bf16x2_bits(p[0], p[1]), bf16x2_bits(p[2], p[3]), bf16x2_bits(p[4], p[5]), bf16x2_bits(p[6], p[7])));
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) {
      acc[qf][hf] *= alpha;
      acc[qf][hf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[hf], pf, acc[qf][hf], 0, 0, 0);
    }
  }
}

template <int HD, int QF, int NW>
__global__ __launch_bounds__(64 * NW) void attention_mfma_kernel(AttnArgs a) {
  constexpr int KS = (HD + 31) / 32;  // 32-wide k steps over the head dim (zero padded)
  constexpr int HF = HD / 16;         // 16-row fragments of the head dim
  __shared__ float red_m[NW][QF * 16];
  __shared__ float red_l[NW][QF * 16];
  __shared__ float red_o[NW][QF * 16][HD + 1];

  const int h = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int S = a.S, Lk = a.Lk, Lp = a.Lp, nh = a.nh;
  const long bh = (long)b * nh + h;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint16_t*)a.q + bh * S * HD, (uint32_t)(S * HD * 2));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint16_t*)a.k + bh * Lp * HD, (uint32_t)(Lp * HD * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint16_t*)a.vt + bh * HD * Lp, (uint32_t)(Lp * HD * 2));
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(a.mask ? a.mask + (long)b * Lk : nullptr, a.mask ? (uint32_t)Lk : 0u);
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)

  // Q^T fragments: lane holds query qf*16 + c16, head dims 32*ks + 8g .. +7
  bf16x8_v qfr[QF][KS];
#pragma unroll
  for (int qf = 0; qf < QF; ++qf)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int qi = qf * 16 + c16, d0 = ks * 32 + g * 8;
      qfr[qf][ks] = __builtin_bit_cast(bf16x8_v, buf_load16(qr, (qi < S && d0 < HD) ? (qi * HD + d0) * 2 : OOB));
    }

  floatx4_t acc[QF][HF];
  float m[QF], l[QF];
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    m[qf] = -INFINITY;
    l[qf] = 0.0f;
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) acc[qf][hf] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // wave w takes tiles w, w + NW, ... two at a time. Both tiles' K/V loads are issued
  // before their mask bytes are read (tiles below ntiles lie inside the padded key rows;
  // a second tile past the end reloads the last one and is not used), so the mask and the
  // tiles cost one memory latency, not two.
  const int ntiles = (Lk + 31) / 32;
  if constexpr (QF >= 3) {
    // many query fragments (long horizons): one tile at a time, so that the registers allow
    // two waves per SIMD
    for (int kt = wave; kt < ntiles; kt += NW) {
      bf16x8_v kf0[2][KS], vf0[HF];
      attn_load_tile<HD>(kr, vr, Lp, kt, g, c16, kf0, vf0);
      asm volatile("" ::: "memory");
      const uint8_t mb0 = buf_load1(mr, kt * 32 + (lane & 31));
      const bool ad0 = lane < 32 && kt * 32 + lane < Lk && (a.mask == nullptr || (mb0 & a.mask_bit) != 0);
      const unsigned long long bal0 = __ballot(ad0);
      const uint32_t bits0 = (uint32_t)(bal0 >> (8 * g)) & 0xFFu;
      if (bal0) attn_tile<HD, QF>(qfr, acc, m, l, kf0, vf0, bits0, (uint32_t)bal0 == 0xFFFFFFFFu, sl2);
    }
  }
  for (int kt = wave; QF < 3 && kt < ntiles; kt += 2 * NW) {
    const int kt2 = kt + NW;
    bf16x8_v kf0[2][KS], vf0[HF], kf1[2][KS], vf1[HF];
    attn_load_tile<HD>(kr, vr, Lp, kt, g, c16, kf0, vf0);
    attn_load_tile<HD>(kr, vr, Lp, min(kt2, ntiles - 1), g, c16, kf1, vf1);
    asm volatile("" ::: "memory");
    // admitted-key bits of the two tiles (lanes < 32: key kt*32 + lane); keys past Lk read 0
    const uint8_t mb0 = buf_load1(mr, kt * 32 + (lane & 31));
    const uint8_t mb1 = buf_load1(mr, kt2 * 32 + (lane & 31));
    const bool ad0 = lane < 32 && kt * 32 + lane < Lk && (a.mask == nullptr || (mb0 & a.mask_bit) != 0);
    const bool ad1 = lane < 32 && kt2 < ntiles && kt2 * 32 + lane < Lk && (a.mask == nullptr || (mb1 & a.mask_bit) != 0);
    const unsigned long long bal0 = __ballot(ad0), bal1 = __ballot(ad1);
    const uint32_t bits0 = (uint32_t)(bal0 >> (8 * g)) & 0xFFu, bits1 = (uint32_t)(bal1 >> (8 * g)) & 0xFFu;
    if (bal0) attn_tile<HD, QF>(qfr, acc, m, l, kf0, vf0, bits0, (uint32_t)bal0 == 0xFFFFFFFFu, sl2);
    if (bal1) attn_tile<HD, QF>(qfr, acc, m, l, kf1, vf1, bits1, (uint32_t)bal1 == 0xFFFFFFFFu, sl2);
  }

  // merge the waves: O^T rows (head dims hf*16 + 4g + i) of query qf*16 + c16
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    if (g == 0) {
      red_m[wave][qf * 16 + c16] = m[qf];
      red_l[wave][qf * 16 + c16] = l[qf];
    }
#pragma unroll
    for (int hf = 0; hf < HF; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_o[wave][qf * 16 + c16][hf * 16 + 4 * g + i] = acc[qf][hf][i];
  }
  __syncthreads();
  uint16_t* o = (uint16_t*)a.o;
  for (int p = t; p < S * HD; p += 64 * NW) {
    const int qi = p / HD, d = p - qi * HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][qi]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = (red_m[w][qi] == -INFINITY) ? 0.0f : exp2f(red_m[w][qi] - M);
        L += red_l[w][qi] * f;
        O += red_o[w][qi][d] * f;
      }
    }
    o[((long)(b * S + qi) * nh + h) * HD + d] = f_to_bf16(L > 0.0f ? O / L : 0.0f);
  }
}

// One wave per (sample, head) pair, four pairs per workgroup: the wave streams every key
// tile of its pair through the online softmax with the next tile's loads in flight, and
// writes its own output (no merge across waves). The admitted-key bitmap of the pair is
// built first (one ballot per 64 keys, loads of 8 words issued together) so that tiles
// without an admitted key are skipped without loading them.
constexpr int AW_MAXWORDS = 8;  // keys per pair <= 512 (one mask byte per lane and word)
constexpr int AW_SETS = 2;  // register sets of the key-tile ring (deeper rings cost occupancy)
template <int HD, int QF, int NS, bool MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attention_wave_kernel(AttnArgs a) {
  constexpr int KS = (HD + 31) / 32, HF = HD / 16;
  __shared__ unsigned long long words_s[4][AW_MAXWORDS];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: descriptors in SGPRs
  const int g = lane >> 4, c16 = lane & 15;
  const int pair = blockIdx.x * 4 + wave;
  if (pair >= a.B * a.nh) return;  // whole wave; the kernel has no workgroup barrier
  const int S = a.S, Lk = a.Lk, Lp = a.Lp, nh = a.nh;
  const int b = pair / nh, h = pair - b * nh;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint16_t*)a.q + (long)pair * S * HD, (uint32_t)(S * HD * 2));
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint16_t*)a.k + (long)pair * Lp * HD, (uint32_t)(Lp * HD * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint16_t*)a.vt + (long)pair * HD * Lp, (uint32_t)(Lp * HD * 2));
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)
  const int ntiles = (Lk + 31) / 32;

  // Every load below is a buffer load issued by every lane (out-of-range lanes read 0)
  // and independent of data loaded before it, so the loads of one phase are in flight
  // together and the compiler's wait counts stay exact.
  // Mask bytes first (the ballots wait for them alone); keys >= Lk read 0.
  uint8_t mb[AW_MAXWORDS];
  if constexpr (MASK) {
    const __amdgpu_buffer_rsrc_t mr = make_rsrc(a.mask + (long)b * Lk, (uint32_t)Lk);
#pragma unroll
    for (int u = 0; u < AW_MAXWORDS; ++u) mb[u] = buf_load1(mr, u * 64 + lane);
  }
  // Q^T fragments: lane holds query qf*16 + c16, head dims 32*ks + 8g .. +7
  bf16x8_v qfr[QF][KS];
#pragma unroll
  for (int qf = 0; qf < QF; ++qf)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int qi = qf * 16 + c16, d0 = ks * 32 + g * 8;
      qfr[qf][ks] = __builtin_bit_cast(bf16x8_v, buf_load16(qr, (qi < S && d0 < HD) ? (qi * HD + d0) * 2 : OOB));
    }
  // the first NS key tiles, before their masks are known (every tile below ntiles lies
  // inside the padded key rows)
  bf16x8_v kf[NS][2][KS], vf[NS][HF];
#pragma unroll
  for (int sidx = 0; sidx < NS; ++sidx) attn_load_tile<HD>(kr, vr, Lp, min(sidx, ntiles - 1), g, c16, kf[sidx], vf[sidx]);

  // admitted-key bitmap: word w holds keys 64w .. 64w+63 (Lk <= 64 * AW_MAXWORDS)
#pragma unroll
  for (int u = 0; u < AW_MAXWORDS; ++u) {
    const int j = u * 64 + lane;
    bool adm;
    if constexpr (MASK) adm = (mb[u] & a.mask_bit) != 0;
    else adm = j < Lk;
    const unsigned long long bal = __ballot(adm);
    if (lane == 0) words_s[wave][u] = bal;
  }
  // 32-bit admitted mask of key tile kt (0 <= kt < ntiles)
  auto tile_mask = [&](int kt) -> uint32_t { return (uint32_t)(words_s[wave][kt >> 1] >> (32 * (kt & 1))); };
  // first and last tile with an admitted key (t1 < 0: none)
  int t0 = ntiles, t1 = -1;
  for (int c0 = 0; c0 < ntiles; c0 += 64) {
    const int kt = c0 + lane;
    const unsigned long long bal = __ballot(kt < ntiles && tile_mask(kt < ntiles ? kt : 0) != 0u);
    if (bal) {
      t0 = min(t0, c0 + (int)__builtin_ctzll(bal));
      t1 = c0 + 63 - (int)__builtin_clzll(bal);
    }
  }

  floatx4_t acc[QF][HF];
  float m[QF], l[QF];
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    m[qf] = -INFINITY;
    l[qf] = 0.0f;
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) acc[qf][hf] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ring of NS register sets over tiles 0 .. t1: set kt % NS holds tile kt when tile kt
  // is processed; after use it is refilled with tile kt + NS, clamped into [t0, t1] (a
  // clamped refill below t0 is replaced before use; one above t1 is never used)
  for (int kt0 = 0; kt0 <= t1; kt0 += NS) {
#pragma unroll
    for (int sidx = 0; sidx < NS; ++sidx) {
      const int kt = kt0 + sidx;
      const uint32_t mt = kt <= t1 ? tile_mask(kt) : 0u;
      if (mt) attn_tile<HD, QF>(qfr, acc, m, l, kf[sidx], vf[sidx], (mt >> (8 * g)) & 0xFFu, mt == 0xFFFFFFFFu, sl2);
      attn_load_tile<HD>(kr, vr, Lp, min(max(kt + NS, t0), t1), g, c16, kf[sidx], vf[sidx]);
    }
  }

  // O^T: lane holds head dims hf*16 + 4g + i of query qf*16 + c16
  uint16_t* o = (uint16_t*)a.o;
#pragma unroll
  for (int qf = 0; qf < QF; ++qf) {
    const int qi = qf * 16 + c16;
    if (qi >= S) continue;
    const float inv = l[qf] > 0.0f ? 1.0f / l[qf] : 0.0f;
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) {
      const floatx4_t v = acc[qf][hf] * inv;
      *(uint2*)(o + ((long)(b * S + qi) * nh + h) * HD + hf * 16 + 4 * g) =
          make_uint2(bf16x2_bits(v[0], v[1]),
                     bf16x2_bits(v[2], v[3]));
    }
  }
}

// 8 waves for small batches with few query fragments (B = 1 latency: more key tiles in
// flight per head); 4 waves otherwise (enough workgroups fill the chip; smaller merge).
template <int HD>
static hipError_t attn_mfma_hd(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.nh, a.B);
  const int qf = (a.S + 15) / 16;
  const bool wide = a.B * a.nh < 512;
  if (a.B * a.nh >= 1024 && a.Lk <= 64 * AW_MAXWORDS && qf <= 2) {
    const dim3 wgrid((a.B * a.nh + 3) / 4);
    if (a.mask) {
      if (qf == 1) hipLaunchKernelGGL((attention_wave_kernel<HD, 1, AW_SETS, true>), wgrid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attention_wave_kernel<HD, 2, AW_SETS, true>), wgrid, dim3(256), 0, s, a);
    } else {
      if (qf == 1) hipLaunchKernelGGL((attention_wave_kernel<HD, 1, AW_SETS, false>), wgrid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((attention_wave_kernel<HD, 2, AW_SETS, false>), wgrid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  switch (qf) {
    case 1:
      if (wide) hipLaunchKernelGGL((attention_mfma_kernel<HD, 1, 8>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((attention_mfma_kernel<HD, 1, 4>), grid, dim3(256), 0, s, a);
      break;
    case 2:
      if (wide) hipLaunchKernelGGL((attention_mfma_kernel<HD, 2, 8>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((attention_mfma_kernel<HD, 2, 4>), grid, dim3(256), 0, s, a);
      break;
    case 3: hipLaunchKernelGGL((attention_mfma_kernel<HD, 3, 4>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attention_mfma_kernel<HD, 4, 4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((attention_mfma_kernel<HD, 5, 4>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, DType t, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.S > AT_SMAX || a.hd > AT_HDMAX || a.S <= 0 || a.Lk <= 0 || a.Lp < a.Lk || (a.Lp % 32) != 0)
    return hipErrorInvalidValue;
  if (t == DT_BF16) {
    switch (a.hd) {
      case 16: return attn_mfma_hd<16>(a, s);
      case 32: return attn_mfma_hd<32>(a, s);
      case 48: return attn_mfma_hd<48>(a, s);
      case 64: return attn_mfma_hd<64>(a, s);
      default: break;
    }
    hipLaunchKernelGGL((attention_valu_kernel<bf16>), dim3(a.nh, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (t == DT_F32) {
    hipLaunchKernelGGL((attention_valu_kernel<float>), dim3(a.nh, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------
// Small kernels
// ------------------------------------------------------------------------------------
__global__ void mask_codes_kernel(const uint8_t* vl_mask, const uint8_t* image_mask, uint8_t* code, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const bool valid = vl_mask ? (vl_mask[i] != 0) : true;
  uint8_t c;
  if (image_mask == nullptr) {
    c = valid ? 3 : 0;
  } else {
    const bool img = image_mask[i] != 0;
    c = (uint8_t)((valid && !img) ? 1 : 0) | (uint8_t)((valid && img) ? 2 : 0);
  }
  code[i] = c;
}

hipError_t launch_mask_codes(const uint8_t* vl_mask, const uint8_t* image_mask, uint8_t* code, int n,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(mask_codes_kernel, dim3((n + 255) / 256), dim3(256), 0, s, vl_mask, image_mask, code, n);
  return hipGetLastError();
}

// Stream compaction of the admitted VL rows: one workgroup of 1024 threads; thread t owns a
// contiguous chunk, chunk counts are scanned in LDS, then every thread writes its indices.
__global__ __launch_bounds__(1024) void compact_rows_kernel(const uint8_t* code, int n, int* idx, int* count) {
  __shared__ int cnt[1024];
  const int t = threadIdx.x;
  const int chunk = (n + 1023) / 1024;
  const int lo = min(n, t * chunk), hi = min(n, lo + chunk);
  int c = 0;
  for (int r = lo; r < hi; ++r) c += code[r] != 0;
  cnt[t] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int v = t >= off ? cnt[t - off] : 0;
    __syncthreads();
    cnt[t] += v;
    __syncthreads();
  }
  int pos = cnt[t] - c;
  for (int r = lo; r < hi; ++r)
    if (code[r] != 0) idx[pos++] = r;
  if (t == 1023) *count = cnt[1023];
}

hipError_t launch_compact_rows(const uint8_t* code, int n, int* idx, int* count, hipStream_t s) {
  hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(1024), 0, s, code, n, idx, count);
  return hipGetLastError();
}

__global__ void sanitize_ids_kernel(const int* ids_in, int* ids_out, uint8_t* bad, int B, int C,
                                    unsigned* bad_count) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int id = ids_in[b];
  const bool ok = id >= 0 && id < C;
  ids_out[b] = ok ? id : 0;
  bad[b] = ok ? 0 : 1;
  if (!ok && bad_count) atomicAdd(bad_count, 1u);
}

hipError_t launch_sanitize_ids(const int* ids_in, int* ids_out, uint8_t* bad, int B, int C, hipStream_t s,
                               unsigned* bad_count) {
  hipLaunchKernelGGL(sanitize_ids_kernel, dim3((B + 255) / 256), dim3(256), 0, s, ids_in, ids_out, bad, B, C,
                     bad_count);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void bucket_ids_kernel(const int* ids, int B, int C, int cap, int* perm,
                                                         int4* chunks, int maxch) {
  extern __shared__ int bsh[];  // count[C], first sample[C + 1], first chunk[C + 1]
  int* cnt = bsh;
  int* first = bsh + C;
  int* cfirst = first + C + 1;
  const int t = threadIdx.x;
  for (int c = t; c < C; c += blockDim.x) cnt[c] = 0;
  __syncthreads();
  for (int b = t; b < B; b += blockDim.x) atomicAdd(&cnt[ids[b]], 1);
  __syncthreads();
  if (t == 0) {
    int f = 0, fc = 0;
    for (int c = 0; c < C; ++c) {
      first[c] = f;
      cfirst[c] = fc;
      f += cnt[c];
      fc += (cnt[c] + cap - 1) / cap;
    }
    first[C] = f;
    cfirst[C] = fc;
  }
  __syncthreads();
  // rank of sample b among the samples of its category (stable order)
  for (int b = t; b < B; b += blockDim.x) {
    const int id = ids[b];
    int rank = 0;
    for (int q = 0; q < b; ++q) rank += ids[q] == id ? 1 : 0;
    perm[first[id] + rank] = b;
  }
  for (int j = t; j < maxch; j += blockDim.x) {
    int4 ch = make_int4(0, 0, 0, 0);
    if (j < cfirst[C]) {
      int lo = 0, hi = C - 1;  // the category whose chunks hold j: last c with cfirst[c] <= j
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (cfirst[mid] <= j) lo = mid;
        else hi = mid - 1;
      }
      const int k = j - cfirst[lo];
      ch = make_int4(lo, first[lo] + k * cap, min(cap, cnt[lo] - k * cap), 0);
    }
    chunks[j] = ch;
  }
}

hipError_t launch_bucket_ids(const int* ids, int B, int C, int cap, int* perm, int4* chunks, hipStream_t s) {
  if (B <= 0 || C <= 0 || cap <= 0) return hipErrorInvalidValue;
  const size_t lds = (size_t)(3 * C + 2) * sizeof(int);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bucket_ids_kernel, dim3(1), dim3(1024), lds, s, ids, B, C, cap, perm, chunks,
                     bucket_max_chunks(B, C, cap));
  return hipGetLastError();
}

__global__ void copy_rows_kernel(const float* src, long src_ld, float* dst, long dst_ld, long dst_gstride,
                                 int dst_row_off, int D) {
  const int b = blockIdx.y;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < D; c += gridDim.x * blockDim.x)
    dst[((long)b * dst_gstride + dst_row_off) * dst_ld + c] = src[(long)b * src_ld + c];
}

hipError_t launch_copy_rows(const float* src, long src_ld, float* dst, long dst_ld, long dst_gstride,
                            int dst_row_off, int B, int D, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3((D + 255) / 256, B), dim3(256), 0, s, src, src_ld, dst, dst_ld,
                     dst_gstride, dst_row_off, D);
  return hipGetLastError();
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy as
// 1, 2, 3", SC 2011): counter (i, call lo, call hi, 0), key = seed; Box-Muller on
// the four 32-bit outputs gives four N(0,1) draws.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = M0 * c[0], hi0 = __umulhi(M0, c[0]);
    const uint32_t lo1 = M1 * c[2], hi1 = __umulhi(M1, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

__global__ void init_noise_kernel(const float* noise, float* x, long n, uint64_t seed, uint64_t counter) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (noise) {
    if (i < n) x[i] = noise[i];
    return;
  }
  const long base = i * 4;
  if (base >= n) return;
  uint32_t c[4] = {(uint32_t)i, (uint32_t)counter, (uint32_t)(counter >> 32), 0u};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  float z[4];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float u1 = ((float)c[2 * p] + 0.5f) * 2.3283064365386963e-10f;
    const float u2 = ((float)c[2 * p + 1] + 0.5f) * 2.3283064365386963e-10f;
    const float r = sqrtf(-2.0f * logf(u1));
    const float th = 6.283185307179586f * u2;
    z[2 * p] = r * cosf(th);
    z[2 * p + 1] = r * sinf(th);
  }
  for (int q = 0; q < 4; ++q)
    if (base + q < n) x[base + q] = z[q];
}

hipError_t launch_init_noise(const float* noise, float* x, long n, uint64_t seed, uint64_t counter, hipStream_t s) {
  const long threads = noise ? n : (n + 3) / 4;
  hipLaunchKernelGGL(init_noise_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, noise, x, n, seed,
                     counter);
  return hipGetLastError();
}

__global__ void output_kernel(const float* x, const uint8_t* mask, const uint8_t* bad, float* out, int B, int per) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)B * per) return;
  const int b = (int)(i / per);
  float v = x[i];
  if (mask) v = mask[i] ? v : 0.0f;
  out[i] = bad[b] ? __int_as_float(0x7fc00000) : v;
}

hipError_t launch_output(const float* x, const uint8_t* mask, const uint8_t* bad, float* out, int B, int per,
                         hipStream_t s) {
  const long n = (long)B * per;
  hipLaunchKernelGGL(output_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, mask, bad, out, B, per);
  return hipGetLastError();
}

struct TauList {
  int v[64];
};

// Timestep sinusoid in double precision (arguments reach ~900 rad), stored as fp32.
__global__ void sinusoid_kernel(TauList tau, int dim, float* tab) {
  const int k = blockIdx.x;
  const int half = dim / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double w = pow(10000.0, -(double)i / (double)half);
    const double arg = (double)tau.v[k] * w;
    tab[(long)k * dim + i] = (float)sin(arg);
    tab[(long)k * dim + half + i] = (float)cos(arg);
  }
}

hipError_t launch_sinusoid(const int* tau_host_k, int K, int dim, float* tab, hipStream_t s) {
  if (K > 64) return hipErrorInvalidValue;
  TauList t;
  for (int k = 0; k < 64; ++k) t.v[k] = k < K ? tau_host_k[k] : 0;
  hipLaunchKernelGGL(sinusoid_kernel, dim3(K), dim3(256), 0, s, t, dim, tab);
  return hipGetLastError();
}

// Flow-matching training ("GR00T model class", Flow matching diffusion, Training; "Model
// architecture", Training objective): per-sample timestep sinusoids, the noisy trajectory
// and the masked squared-error loss.
__global__ void sinusoid_t_kernel(const float* t, int buckets, int dim, float* tab) {
  const int b = blockIdx.x;
  const int tau = (int)floorf(t[b] * (float)buckets);  // the bucket, decided in fp32
  const int half = dim / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double w = pow(10000.0, -(double)i / (double)half);
    const double arg = (double)tau * w;
    tab[(long)b * dim + i] = (float)sin(arg);
    tab[(long)b * dim + half + i] = (float)cos(arg);
  }
}

hipError_t launch_sinusoid_t(const float* t, int n, int buckets, int dim, float* tab, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sinusoid_t_kernel, dim3(n), dim3(256), 0, s, t, buckets, dim, tab);
  return hipGetLastError();
}

__global__ void flow_interp_kernel(const float* a, const float* z, const float* t, float* x, int per, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float tb = t[i / per];
  x[i] = (1.0f - tb) * z[i] + tb * a[i];
}

hipError_t launch_flow_interp(const float* actions, const float* noise, const float* t, float* x, int B, int per,
                              hipStream_t s) {
  const long n = (long)B * per;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(flow_interp_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, actions, noise, t, x,
                     per, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void masked_mse_kernel(const float* vp, const float* a, const float* z,
                                                          const uint8_t* mask, const uint8_t* bad, int B, long n,
                                                          float* loss) {
  __shared__ double sn[1024], sd[1024];
  const int t = threadIdx.x;
  double num = 0.0, den = 0.0;
  for (long i = t; i < n; i += 1024) {  // each thread in index order, then a fixed tree
    const double m = mask ? (double)mask[i] : 1.0;
    const double d = (double)vp[i] - ((double)a[i] - (double)z[i]);
    num += m * d * d;
    den += m;
  }
  sn[t] = num;
  sd[t] = den;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) {
      sn[t] += sn[t + w];
      sd[t] += sd[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    int anybad = 0;
    for (int b = 0; b < B; ++b) anybad |= bad ? bad[b] : 0;
    loss[0] = anybad ? __builtin_nanf("") : (float)(sn[0] / (sd[0] + 1e-6));
  }
}

hipError_t launch_masked_mse(const float* v_pred, const float* actions, const float* noise, const uint8_t* mask,
                             const uint8_t* bad, int B, int per, float* loss, hipStream_t s) {
  if (B <= 0 || per <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(masked_mse_kernel, dim3(1), dim3(1024), 0, s, v_pred, actions, noise, mask, bad, B,
                     (long)B * per, loss);
  return hipGetLastError();
}

// W8A8: per-row e4m3 inputs of the e4m3-weight GEMMs ("fp8a8" mode). One wave per row of bf16
// x: scale[r] = amax_r / 448 (1 for an all-zero row), q[r][k] = e4m3(x[r][k] / scale[r]); both
// divisions correctly rounded in fp32. The codes come from the gfx950 conversion instruction
// (v_cvt_pk_fp8_f32, round to nearest even): it equals the nearest-even OCP e4m3 code, sign
// included, on every fp32 value of magnitude up to 460 (checked exhaustively on the GPU), and the
// quotients stay below 448 * (1 + 2^-23). Rows r >= *rows_dev (when given) are skipped.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, long ldx, int rows, int K,
                                                         uint8_t* __restrict__ q, long ldq, float* __restrict__ scale,
                                                         const int* rows_dev) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows || (rows_dev && row >= *rows_dev)) return;
  const uint16_t* xr = x + (long)row * ldx;
  float amax = 0.0f;
  for (int k = 8 * lane; k < K; k += 512) {  // 8 values (16 bytes) per lane and step
    const uint4 v = *(const uint4*)(xr + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f(w[i] & 0xFFFFu)), fabsf(bf16_to_f(w[i] >> 16))));
  }
  amax = wave_max(amax);
  const float sc = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (lane == 0) scale[row] = sc;
  uint8_t* qr = q + (long)row * ldq;
  for (int k = 8 * lane; k < K; k += 512) {
    const uint4 v = *(const uint4*)(xr + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __fdiv_rn(bf16_to_f(w[i] & 0xFFFFu), sc);
      f[2 * i + 1] = __fdiv_rn(bf16_to_f(w[i] >> 16), sc);
    }
    int c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    c0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], c0, true);
    int c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    c1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], c1, true);
    *(uint2*)(qr + k) = make_uint2((uint32_t)c0, (uint32_t)c1);
  }
}

hipError_t launch_quant_rows(const void* x, long ldx, int rows, int K, uint8_t* q, long ldq, float* scale,
                             hipStream_t s, const int* rows_dev) {
  if (rows <= 0) return hipSuccess;
  if ((K % 8) != 0 || (ldx % 8) != 0 || (ldq % 8) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, (const uint16_t*)x, ldx, rows, K, q,
                     ldq, scale, rows_dev);
  return hipGetLastError();
}

__global__ void silu_kernel(const float* x, float* y, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = silu_f(x[i]);
}

hipError_t launch_silu(const float* x, float* y, long n, hipStream_t s) {
  hipLaunchKernelGGL(silu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

__global__ void convert_kernel(const float* x, bf16* y, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) st(y + i, x[i]);
}

hipError_t launch_convert(const float* x, void* y, DType yt, long n, hipStream_t s) {
  if (yt != DT_BF16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(convert_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, (bf16*)y, n);
  return hipGetLastError();
}

}  // namespace gr00t

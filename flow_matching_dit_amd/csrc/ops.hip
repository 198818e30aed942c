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
                                                        const float* __restrict__ ada) {
  constexpr int MAXPER = 32;  // D <= 2048
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const TX* xr = x + (long)row * ldx;
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
                            const float* gamma, const float* beta, const float* ada, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (D > 2048) return hipErrorInvalidValue;
  dim3 grid((rows + 3) / 4);
  if (xt == DT_F32 && yt == DT_F32)
    hipLaunchKernelGGL((layernorm_kernel<float, float>), grid, dim3(256), 0, s, (const float*)x, ldx, (float*)y, ldy,
                       rows, D, gamma, beta, ada);
  else if (xt == DT_F32 && yt == DT_BF16)
    hipLaunchKernelGGL((layernorm_kernel<float, bf16>), grid, dim3(256), 0, s, (const float*)x, ldx, (bf16*)y, ldy,
                       rows, D, gamma, beta, ada);
  else if (xt == DT_BF16 && yt == DT_BF16)
    hipLaunchKernelGGL((layernorm_kernel<bf16, bf16>), grid, dim3(256), 0, s, (const bf16*)x, ldx, (bf16*)y, ldy,
                       rows, D, gamma, beta, ada);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Attention on the vector ALUs: one workgroup per (head, sample); keys streamed in
// chunks of 64 through LDS with an online (running max / running sum) softmax in
// fp32. Self-attention blocks pass the S state+action tokens as keys; cross-attention
// blocks pass the cached VL keys/values with the block's key mask
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
  const int S = a.S, hd = a.hd, Lk = a.Lk, nh = a.nh;
  const T* q = (const T*)a.q + (long)(b * nh + h) * S * hd;
  const T* k = (const T*)a.k + (long)(b * nh + h) * Lk * hd;
  const T* v = (const T*)a.v + (long)(b * nh + h) * Lk * hd;
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
      Vs[jj][d] = in ? ld(v + (long)(j0 + jj) * hd + d) : 0.0f;
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

hipError_t launch_attention(const AttnArgs& a, DType t, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.S > AT_SMAX || a.hd > AT_HDMAX || a.S <= 0 || a.Lk <= 0) return hipErrorInvalidValue;
  dim3 grid(a.nh, a.B);
  if (t == DT_F32)
    hipLaunchKernelGGL((attention_valu_kernel<float>), grid, dim3(256), 0, s, a);
  else if (t == DT_BF16)
    hipLaunchKernelGGL((attention_valu_kernel<bf16>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
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

__global__ void sanitize_ids_kernel(const int* ids_in, int* ids_out, uint8_t* bad, int B, int C) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int id = ids_in[b];
  const bool ok = id >= 0 && id < C;
  ids_out[b] = ok ? id : 0;
  bad[b] = ok ? 0 : 1;
}

hipError_t launch_sanitize_ids(const int* ids_in, int* ids_out, uint8_t* bad, int B, int C, hipStream_t s) {
  hipLaunchKernelGGL(sanitize_ids_kernel, dim3((B + 255) / 256), dim3(256), 0, s, ids_in, ids_out, bad, B, C);
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

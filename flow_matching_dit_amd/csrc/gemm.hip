// GEMMs of the action head for gfx950.
//
//  * gemm_dma_kernel: bf16 activations x bf16 weights on the matrix cores
//    (v_mfma_f32_16x16x32_bf16), fp32 accumulation. Tiles of A [BM x 64] and
//    W [BN x 64] go from memory straight into LDS (buffer_load ... lds) through a
//    ring of 3 stages, so two tiles of loads are in flight while one is multiplied.
//    e4m3 weights take the same kernel with their bytes in LDS, each fragment decoded
//    to bf16 (exactly) after its LDS read; the per-column scale is applied in the
//    epilogue.
//  * gemm_a8_kernel: e4m3 activations x e4m3 weights (W8A8) on the fp8 matrix
//    instruction (v_mfma_f32_16x16x128_f8f6f4), with per-row and per-column scales.
//    Both load through buffer descriptors, so rows or k beyond the matrix read as
//    zero without branches.
//    The MFMA computes C^T = W A^T per 16x16 fragment, so every lane ends with four
//    consecutive output columns of one row: the epilogue stores 8 or 16 bytes per lane.
//    Workgroups are numbered so that consecutive tiles share weight columns and land
//    on the same XCD (workgroups are dealt round-robin over the 8 XCDs).
//    Optional split-K writes fp32 partial sums that the next LayerNorm reduces in a
//    fixed order (deterministic).
//  * gemm_valu_kernel: fp32 FMA on the vector ALUs for any (A, W) storage types.
//    Serves the fp32 path, the input-independent tables and the per-embodiment
//    linears whose K or N is the small action/state width.
//
// Both read a group/category description (GemmArgs), so one launch covers the
// per-sample weight gather of the per-embodiment linear (the batched product over
// W[ids] on the architecture page, "Embodiment-specific projectors"), and finish
// with a fused epilogue (bias, activation, residual add, head-major scatter, Euler).
#include <algorithm>
#include <type_traits>

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

// Epilogue of NV consecutive columns n .. n+NV-1 of row r in group g (values already
// scaled and biased). NV is 1 (VALU kernel) or 4 (MFMA kernel).
template <int EK, int NV>
__device__ __forceinline__ void epi_store(const Epi& e, int g, int r, int n, float (&v)[NV], int cat, int split) {
  if (e.add_tab) {
#pragma unroll
    for (int q = 0; q < NV; ++q) v[q] += e.add_tab[(long)(e.add_by_group ? g : cat) * e.add_cstride + n + q];
  }
  if (EK != EPI_PARTIAL) {
#pragma unroll
    for (int q = 0; q < NV; ++q) v[q] = apply_act(e.act, v[q]);
  }
  const long row0 = (long)g * e.out_gstride + e.out_row_off + r;
  if (EK == EPI_STORE) {
    const long row = row0;
    const long idx = row * e.out_ld + n;
    if (e.out_f32) {
      float* p = (float*)e.out + idx;
      if (NV == 4) *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
      else
#pragma unroll
        for (int q = 0; q < NV; ++q) p[q] = v[q];
    } else {
      uint16_t* p = (uint16_t*)e.out + idx;
      if (NV == 4) {
        *(uint2*)p = make_uint2(bf16x2_bits(v[0], v[1]),
                                bf16x2_bits(v[2], v[3]));
      } else {
#pragma unroll
        for (int q = 0; q < NV; ++q) p[q] = f_to_bf16(v[q]);
      }
    }
  } else if (EK == EPI_RESID_ADD || EK == EPI_EULER) {
    const long row = row0;
    float* p = (float*)e.out + row * e.out_ld + n;
    const float s = (EK == EPI_EULER) ? e.dt : 1.0f;
    if (NV == 4) {
      float4 o = *(float4*)p;
      o.x += s * v[0];
      o.y += s * v[1];
      o.z += s * v[2];
      o.w += s * v[3];
      *(float4*)p = o;
    } else {
#pragma unroll
      for (int q = 0; q < NV; ++q) p[q] = p[q] + s * v[q];
    }
  } else if (EK == EPI_PARTIAL) {
    const long row = row0;
    float* p = (float*)e.out + (long)split * e.split_stride + row * e.out_ld + n;
    if (NV == 4) *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    else
#pragma unroll
      for (int q = 0; q < NV; ++q) p[q] = v[q];
  } else {  // EPI_HEADS: NV consecutive columns stay inside one head (hd % 4 == 0)
    const long row = e.row_map ? (long)e.row_map[row0] : row0;
    const int sec = n / e.width;
    const int which = sec % e.nwhich;
    const int layer = sec / e.nwhich;
    const int c = n - sec * e.width;
    const int head = c / e.hd;
    const int d = c - head * e.hd;
    const int b = (int)(row / e.pos_per_b);
    const int pos = (int)(row - (long)b * e.pos_per_b);
    const long bh = (long)b * e.nh + head;
    const long ps = e.pstride[which];
    const long base = (long)layer * e.layer_stride[which];
    if (e.transposed[which]) {  // [pos / 32][hd][pos % 32] per (sample, head)
      const long idx = base + bh * e.hd * ps + (long)(pos >> 5) * e.hd * 32 + d * 32 + (pos & 31);
      if (e.out_f32) {
#pragma unroll
        for (int q = 0; q < NV; ++q) ((float*)e.heads[which])[idx + q * 32] = v[q];
      } else {
#pragma unroll
        for (int q = 0; q < NV; ++q) ((uint16_t*)e.heads[which])[idx + q * 32] = f_to_bf16(v[q]);
      }
    } else {
      const long idx = base + (bh * ps + pos) * e.hd + d;
      if (e.out_f32) {
        float* p = (float*)e.heads[which] + idx;
#pragma unroll
        for (int q = 0; q < NV; ++q) p[q] = v[q];
      } else {
        uint16_t* p = (uint16_t*)e.heads[which] + idx;
        if (NV == 4) {
          *(uint2*)p = make_uint2(bf16x2_bits(v[0], v[1]),
                                  bf16x2_bits(v[2], v[3]));
        } else {
#pragma unroll
          for (int q = 0; q < NV; ++q) p[q] = f_to_bf16(v[q]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Vector-ALU GEMM: 64 x 64 tile, 256 threads, 4 x 4 outputs per thread.
// ------------------------------------------------------------------------------------
template <typename TA, typename TW, int EK>
__global__ __launch_bounds__(256) void gemm_valu_kernel(GemmArgs a, Epi e) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Ws[BK][BN + 4];
  const int g = blockIdx.z;
  const int cat = a.ids ? a.ids[g] : 0;
  const int r0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  if (a.rows_dev) {
    const int rr = min(a.rows, *a.rows_dev);
    if (r0 >= rr) return;
    a.rows = rr;
  }
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
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (r < a.rows && n < a.N) {
        float v[1] = {acc[i][j]};
        if (a.wscale) v[0] *= a.wscale[(long)cat * a.s_cstride + n];
        if (a.bias) v[0] += a.bias[(long)cat * a.b_cstride + n];
        epi_store<EK, 1>(e, g, r, n, v, cat, 0);
      }
    }
  }
}

// Vector-ALU GEMM for at most 32 rows: the 64 x 64 tile leaves a handful of workgroups each
// walking all of K. Here a workgroup owns 4 output columns and its 256 threads split K into
// 64 slices (thread t: column t % 4, k = 4 (t / 4) + 256 i .. +3, loaded as one vector, every
// row in registers); the slices' partial sums are added in slice order through LDS. Needs
// K and lda multiples of 4 (vector loads).
constexpr int VS_COLS = 4, VS_SLICES = 64, VS_ROWS = 32;
template <typename T>
__device__ __forceinline__ void ld4(const T* p, float (&v)[4]);
template <>
__device__ __forceinline__ void ld4<float>(const float* p, float (&v)[4]) {
  const float4 f = *(const float4*)p;
  v[0] = f.x;
  v[1] = f.y;
  v[2] = f.z;
  v[3] = f.w;
}
template <>
__device__ __forceinline__ void ld4<bf16>(const bf16* p, float (&v)[4]) {
  const uint2 u = *(const uint2*)p;
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
template <typename TA, typename TW, int EK>
__global__ __launch_bounds__(256) void gemm_valu_skinny_kernel(GemmArgs a, Epi e) {
  __shared__ float red[VS_SLICES][VS_ROWS][VS_COLS + 1];
  if (a.rows_dev) a.rows = min(a.rows, *a.rows_dev);
  const int g = blockIdx.z;
  const int cat = a.ids ? a.ids[g] : 0;
  const int t = threadIdx.x, c = t % VS_COLS, sl = t / VS_COLS;
  const int n = blockIdx.x * VS_COLS + c;
  const TA* A = (const TA*)a.A + ((long)g * a.a_gstride + a.a_row_off) * a.lda;
  const TW* W = (const TW*)a.W + (long)cat * a.w_cstride;
  float acc[VS_ROWS];
#pragma unroll
  for (int r = 0; r < VS_ROWS; ++r) acc[r] = 0.0f;
  if (n < a.N) {
    const TW* wr = W + (long)n * a.K;
    for (int k0 = 4 * sl; k0 < a.K; k0 += 4 * VS_SLICES) {
      float wv[4];
      ld4(wr + k0, wv);
#pragma unroll
      for (int r = 0; r < VS_ROWS; ++r) {
        if (r >= a.rows) break;
        float av[4];
        ld4(A + (long)r * a.lda + k0, av);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[r] = fmaf(av[q], wv[q], acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < VS_ROWS; ++r) red[sl][r][c] = acc[r];
  __syncthreads();
  for (int p = t; p < a.rows * VS_COLS; p += 256) {
    const int r = p / VS_COLS, cc = p % VS_COLS, nn = blockIdx.x * VS_COLS + cc;
    if (nn >= a.N) continue;
    float s = 0.0f;
    for (int q = 0; q < VS_SLICES; ++q) s += red[q][r][cc];
    float v[1] = {s};
    if (a.wscale) v[0] *= a.wscale[(long)cat * a.s_cstride + nn];
    if (a.bias) v[0] += a.bias[(long)cat * a.b_cstride + nn];
    epi_store<EK, 1>(e, g, r, nn, v, cat, 0);
  }
}

// ------------------------------------------------------------------------------------
// MFMA GEMM
// ------------------------------------------------------------------------------------

// The two e4m3 codes in the low 16 bits of w -> two bf16 (bits). One gfx950 conversion
// instruction (OCP e4m3fn, scale 1: exact, every e4m3 value is a bf16 value; measured equal
// to the bitwise decode for all 254 finite codes); the bitwise decode it replaces took about
// ten VALU operations per value, which made the e4m3 GEMMs VALU-bound.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// Map the linear workgroup id to (tile_m, tile_n): ids are first regrouped so that each
// XCD (id % 8) receives a contiguous range, then ranges walk GM m-tiles fastest so that
// neighbouring workgroups reuse the same weight columns from the XCD's L2.
template <int GM>
__device__ __forceinline__ void tile_of(int nm, int nn, int& tm, int& tn) {
  const int nb = nm * nn;
  const int id = blockIdx.x;
  // bijective regrouping: XCD x (= id % 8) owns the contiguous range starting at
  // x * q + min(x, r), where q = nb / 8 and r = nb % 8
  const int q = nb >> 3, r = nb & 7;
  const int x = id & 7;
  const int lid = x * q + min(x, r) + (id >> 3);
  const int group = lid / (GM * nn);
  const int first = group * GM;
  const int gm = min(GM, nm - first);
  const int in = lid - group * GM * nn;
  tm = first + in % gm;
  tn = in / gm;
}

// Split-K launches (grid nb x 1 x S, S dividing 8, nb * S a multiple of 8): workgroups are
// dealt round-robin over the 8 XCDs in dispatch order (x fastest, then z), so XCD
// id % 8 is given the K-slice split = xcd / (8 / S) and a contiguous run of that slice's
// tiles. Each XCD then reads only its slice of A (with the plain mapping every XCD reads
// all of A once per slice). Bijective: split s takes positions [0, nb) from its 8 / S XCDs.
template <int GM>
__device__ __forceinline__ void split_tile_of(int nm, int nn, int S, int& tm, int& tn, int& split) {
  const int nb = nm * nn;
  const int id = (int)blockIdx.x + nb * (int)blockIdx.z;
  const int xcd = id & 7, slot = id >> 3;
  const int nslots = (nb * S) >> 3;
  const int xps = 8 / S;
  split = xcd / xps;
  const int lid = (xcd % xps) * nslots + slot;
  const int group = lid / (GM * nn);
  const int first = group * GM;
  const int gm = min(GM, nm - first);
  const int in = lid - group * GM * nn;
  tm = first + in % gm;
  tn = in / gm;
}

// Epilogue of the MFMA tile kernels: acc[i][j][q] holds row
// r0 + wm*TM + i*16 + lane%16 and column n0 + wn*TN + j*16 + 4*(lane/16) + q.
// res (EPI_RESID_ADD only, may be null): the residual values of acc's positions, loaded by
// the caller ahead of time; the epilogue then stores res + v without reading the output.
template <int BM, int BN, int WM, int WN, int EK>
__device__ __forceinline__ void mfma_epilogue(const GemmArgs& a, const Epi& e,
                                              const floatx4_t (&acc)[BM / WM / 16][BN / WN / 16], int g, int cat,
                                              int split, int r0, int n0, int wm, int wn, int lane,
                                              const float4* res = nullptr, int bfirst = 0, int brows = 1) {
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  const bool add_bias = (EK != EPI_PARTIAL) || split == 0;
  if constexpr (EK == EPI_HEADS) {
    // head-major scatter: the element offset splits into a row part (sample, position)
    // and a column part (section, head, head dim); both are decomposed once per fragment
    int rb[FM], rp[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = r0 + wm * TM + i * 16 + (lane & 15);
      const long row = r < a.rows ? (e.row_map ? (long)e.row_map[r] : (long)r) : 0;
      rb[i] = (int)(row / e.pos_per_b);
      rp[i] = (int)(row - (long)rb[i] * e.pos_per_b);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + j * 16 + (lane >> 4) * 4;
      if (n >= a.N) continue;
      const int sec = n / e.width;
      const int which = sec % e.nwhich;
      const int layer = sec / e.nwhich;
      const int c = n - sec * e.width;
      const int head = c / e.hd;
      const int d = c - head * e.hd;
      const long ps = e.pstride[which];
      const bool tr = e.transposed[which] != 0;
      // transposed: [pos / 32][hd][pos % 32] per (sample, head); else [pos][hd]
      const long colpart = (long)layer * e.layer_stride[which] + (long)head * ps * e.hd + (tr ? d * 32 : d);
      const long bstride = (long)e.nh * ps * e.hd;  // elements per sample in either layout
      float sc[4], bi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sc[q] = a.wscale ? a.wscale[(long)cat * a.s_cstride + n + q] : 1.0f;
        bi[q] = a.bias ? a.bias[(long)cat * a.b_cstride + n + q] : 0.0f;
      }
      uint16_t* base16 = (uint16_t*)e.heads[which];
      float* base32 = (float*)e.heads[which];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = r0 + wm * TM + i * 16 + (lane & 15);
        if (r >= a.rows) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = apply_act(e.act, acc[i][j][q] * sc[q] + bi[q]);
        const long idx = colpart + (long)rb[i] * bstride + (tr ? (long)(rp[i] >> 5) * e.hd * 32 + (rp[i] & 31) : (long)rp[i] * e.hd);
        if (tr) {
          if (e.out_f32) {
#pragma unroll
            for (int q = 0; q < 4; ++q) base32[idx + q * 32] = v[q];
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) base16[idx + q * 32] = f_to_bf16(v[q]);
          }
        } else if (e.out_f32) {
          *(float4*)(base32 + idx) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          *(uint2*)(base16 + idx) = make_uint2(bf16x2_bits(v[0], v[1]),
                                               bf16x2_bits(v[2], v[3]));
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = n0 + wn * TN + j * 16 + (lane >> 4) * 4;
      if (n >= a.N) continue;
      float sc[4], bi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sc[q] = a.wscale ? a.wscale[(long)cat * a.s_cstride + n + q] : 1.0f;
        bi[q] = (a.bias && add_bias) ? a.bias[(long)cat * a.b_cstride + n + q] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = r0 + wm * TM + i * 16 + (lane & 15);
        if (r < a.rows) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[i][j][q] * sc[q] + bi[q];
          if (EK == EPI_RESID_ADD && res != nullptr && e.add_tab == nullptr && e.act == ACT_NONE) {
            const float4 o = res[i * FN + j];
            *(float4*)((float*)e.out + ((long)g * e.out_gstride + e.out_row_off + r) * e.out_ld + n) =
                make_float4(o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]);
          } else if (a.chunks) {  // category bucket: row r % brows of sample perm[first + r / brows]
            epi_store<EK, 4>(e, a.perm[bfirst + r / brows], r % brows, n, v, cat, split);
          } else {
            epi_store<EK, 4>(e, g, r, n, v, cat, split);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// bf16 x bf16 MFMA GEMM whose tiles go straight from memory into LDS
// (buffer_load_dwordx4 ... lds, gfx950), through a ring of ST stages: the loads of
// tile kt + ST - 1 are issued while tile kt is multiplied, so a load has ST - 1 tiles
// of MFMAs to arrive, and no staging registers are needed. A wave's load instruction
// writes 64 consecutive 16-byte LDS chunks (lane l -> chunk l), so the layout is chosen
// through the global address each lane reads.
//  * BK = 64 (128-byte rows): row r keeps its k-chunk c at chunk position c ^ ((r / 2) % 8).
//  * BK = 32 (64-byte rows): each block of 16 rows (1 KB, exactly what one MFMA fragment
//    read covers) is held as 8 lines of 128 bytes; line L holds rows L and L + 8, and the
//    chunk h = (row / 8) + 2 * c of either row sits at position h ^ L of the line.
// Both keep every fragment read free of LDS bank conflicts (the plain row-major XOR for
// 64-byte rows measured half of all LDS cycles as conflicts).
// Accumulation order: k-tiles in order, 32 k per MFMA.
// ------------------------------------------------------------------------------------
// Waits until at most N vector-memory operations of this wave are in flight and all its
// LDS reads have completed, then meets the workgroup barrier. One asm statement, so the
// compiler moves no LDS access across it.
// 16 bytes per lane from the buffer at byte offset off into LDS at lds + 16 * lane
// (lds must be the same for the whole wave).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int V>
using ic = std::integral_constant<int, V>;

// XOR mask of the 16-byte chunk position of e4m3 weight row r (CW chunks per row): with it
// the 8-byte fragment reads of 16 consecutive rows by 32 lanes touch 64 distinct banks.
template <int CW>
__device__ __forceinline__ int wswz8(int r) { return CW == 4 ? (r >> 2) & 3 : (r >> 3) & 1; }

// Eight e4m3 codes -> eight bf16 (exact), four gfx950 conversion instructions.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint2 w) {
  const uint32_t v0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
  const uint32_t v1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
  const uint32_t v2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
  const uint32_t v3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, make_uint4(v0, v1, v2, v3));
}

// XOR mask of the k-chunk position of tile row r (r % 16 given) for 128-byte rows.
__device__ __forceinline__ int kswz64(int r) { return (r >> 1) & 7; }

// f(ic<0>{}), f(ic<1>{}), ..., f(ic<N - 1>{}) in order (compile-time indices).
template <typename F, int... I>
__device__ __forceinline__ void for_seq_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(ic<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void for_seq(F&& f) {
  for_seq_impl(f, std::make_integer_sequence<int, N>{});
}

// W8: the weights are e4m3 bytes [N][K] (one fp32 scale per column, applied in the epilogue).
// Their tiles go into LDS as bytes (CW 16-byte chunks per BK-byte row) and each 8-value
// fragment is decoded to bf16 after its LDS read (four conversion instructions). When a stage
// has fewer weight load instructions than waves, the waves without one load out of range
// (zeros, no memory traffic) into a spare chunk after the stage, so that every wave issues
// the same loads and the wait counts stay exact.
template <int BM, int BN, int WM, int WN, int BK, int ST, int EK, int GM, bool W8 = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(GemmArgs a, Epi e) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int CPR = BK / 8;       // 16-byte chunks per bf16 tile row
  constexpr int RPI = 64 / CPR;     // tile rows per wave load instruction
  constexpr int CW = W8 ? BK / 16 : CPR, RW = 64 / CW;  // weight rows: chunks per row, rows per instruction
  constexpr int NWI = BN / RW;      // weight load instructions per stage
  constexpr int A_I = BM / (RPI * NW), B_I = W8 ? (NWI + NW - 1) / NW : BN / (RPI * NW);
  static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
  static_assert(A_I * RPI * NW == BM && (W8 ? NWI * RW == BN : B_I * RPI * NW == BN),
                "tile rows must split evenly over the waves");
  static_assert(FM >= 1 && FN >= 1, "tile shape");
  static_assert(ST >= 2 && ST <= 6, "2 to 6 stages");
  constexpr int PER_STAGE = A_I + B_I;
  static_assert(PER_STAGE * (ST - 1) < 64, "vmcnt range");

  // One array per stage: the compiler's wait-count tracking then knows that loads into
  // one stage do not alias reads of another (one shared ring would make every LDS read
  // wait for all loads in flight).
  __shared__ __attribute__((aligned(1024))) uint16_t As0[BM * BK], As1[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t As2[ST > 2 ? BM * BK : 8], As3[ST > 3 ? BM * BK : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t As4[ST > 4 ? BM * BK : 8], As5[ST > 5 ? BM * BK : 8];
  constexpr int SB = W8 ? (BN * BK + 1024) / 2 : BN * BK;  // weight stage, 16-bit units (e4m3: bytes + spare)
  __shared__ __attribute__((aligned(1024))) uint16_t Bs0[SB], Bs1[SB];
  __shared__ __attribute__((aligned(1024))) uint16_t Bs2[ST > 2 ? SB : 8], Bs3[ST > 3 ? SB : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t Bs4[ST > 4 ? SB : 8], Bs5[ST > 5 ? SB : 8];
  auto stage_a = [&](auto st) -> uint16_t* {
    constexpr int V = decltype(st)::value;
    if constexpr (V == 0) return As0;
    else if constexpr (V == 1) return As1;
    else if constexpr (V == 2) return As2;
    else if constexpr (V == 3) return As3;
    else if constexpr (V == 4) return As4;
    else return As5;
  };
  auto stage_b = [&](auto st) -> uint16_t* {
    constexpr int V = decltype(st)::value;
    if constexpr (V == 0) return Bs0;
    else if constexpr (V == 1) return Bs1;
    else if constexpr (V == 2) return Bs2;
    else if constexpr (V == 3) return Bs3;
    else if constexpr (V == 4) return Bs4;
    else return Bs5;
  };

  if (a.rows_dev) {
    a.rows = min(a.rows, *a.rows_dev);
    if ((int)blockIdx.x >= ((a.rows + BM - 1) / BM) * ((a.N + BN - 1) / BN)) return;
  }
  const int nm = (a.rows + BM - 1) / BM, nn = (a.N + BN - 1) / BN;
  int tm, tn, split;
  if (gridDim.z > 1 && gridDim.y == 1 && (8 % gridDim.z) == 0 && ((nm * nn * (int)gridDim.z) & 7) == 0) {
    split_tile_of<GM>(nm, nn, (int)gridDim.z, tm, tn, split);
  } else {
    tile_of<GM>(nm, nn, tm, tn);
    split = blockIdx.z;
  }
  const int g = blockIdx.y;
  int cat = a.ids ? a.ids[g] : 0;
  const int r0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * a.k_per_split;
  const int kend = min(a.K, kbeg + a.k_per_split);

  const uint16_t* A = (const uint16_t*)a.A + ((long)g * a.a_gstride + a.a_row_off) * a.lda;
  // category bucket: the chunk's samples, their rows addressed from the start of A
  int bfirst = 0;
  const int brows = a.rows;  // rows per sample
  if (a.chunks) {
    const int4 ch = a.chunks[g];
    if (ch.z <= 0) return;   // an unused chunk (the whole workgroup leaves before any load)
    cat = ch.x;
    bfirst = ch.y;
    a.rows = ch.z * brows;
    A = (const uint16_t*)a.A;
  }
  // element offset of row r of this group (bucket: row r % brows of sample perm[first + r / brows])
  auto a_row = [&](int r) -> long {
    if (!a.chunks) return (long)r * a.lda;
    const int smp = a.perm[bfirst + r / brows];
    return ((long)smp * a.a_gstride + a.a_row_off + r % brows) * a.lda;
  };
  const uint16_t* W = (const uint16_t*)a.W + (long)cat * a.w_cstride;
  const __amdgpu_buffer_rsrc_t ra_rsrc =
      make_rsrc(A, (uint32_t)(a.chunks ? a.map_bytes : (long)a.rows * a.lda * 2));
  const __amdgpu_buffer_rsrc_t rw_rsrc = make_rsrc(W, (uint32_t)((long)a.N * a.K * (W8 ? 1 : 2)));

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave / WN, wn = wave % WN;

  // This lane's chunk in load instruction i (RPI tile rows from row (wave * X_I + i) * RPI):
  // BK = 64: row lane / 8 of the block, k-chunk (lane % 8) ^ ((row / 2) % 8);
  // BK = 32: line L = lane / 8, h = (lane % 8) ^ L, row L + 8 * (h % 2), k-chunk h / 2.
  const int lrow = BK == 32 ? ((lane >> 3) | (((lane & 7) ^ (lane >> 3)) & 1) << 3) : lane / CPR;
  const int lkc = BK == 32 ? (((lane & 7) ^ (lane >> 3)) >> 1) : lane % CPR;
  int aoff[A_I], boff[B_I], akc[A_I], bkc[B_I];
#pragma unroll
  for (int i = 0; i < A_I; ++i) {
    const int row = (wave * A_I + i) * RPI + lrow;
    aoff[i] = (r0 + row < a.rows) ? (int)(a_row(r0 + row) * 2) : OOB;
    if constexpr (BK == 32) akc[i] = lkc * 8;
    else akc[i] = (lkc ^ kswz64(row & 15)) * 8;
  }
  int bdst[B_I];
#pragma unroll
  for (int i = 0; i < B_I; ++i) {
    if constexpr (W8) {
      // e4m3 row r keeps 16-byte chunk c at position c ^ wswz8(r): the 16-row fragment reads
      // (8 bytes per lane) then fall on distinct banks
      const int ii = i * NW + wave, row = ii * RW + lane / CW;
      boff[i] = (ii < NWI && n0 + row < a.N) ? (n0 + row) * a.K : OOB;
      bkc[i] = ((lane % CW) ^ wswz8<CW>(row)) * 16;  // element (= byte) offset in the k-tile
      bdst[i] = min(ii, NWI) * 512;
    } else {
      const int row = (wave * B_I + i) * RPI + lrow;
      boff[i] = (n0 + row < a.N) ? (n0 + row) * a.K * 2 : OOB;
      if constexpr (BK == 32) bkc[i] = lkc * 8;
      else bkc[i] = (lkc ^ kswz64(row & 15)) * 8;
      bdst[i] = (wave * B_I + i) * 64 * 8;
    }
  }
  // Loads of k-tile kt into stage st. Every step issues its loads, also past the last
  // k-tile (those read out of range: zeros, no memory traffic), so the number of loads
  // in flight is the same at every step.
  auto issue = [&](auto st, int kt) {
    uint16_t* sa = stage_a(st);
    uint16_t* sb = stage_b(st);
    const int k0 = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < A_I; ++i)
      dma16(ra_rsrc, sa + (wave * A_I + i) * 64 * 8,
            (k0 + akc[i] < kend && aoff[i] != OOB) ? aoff[i] + (k0 + akc[i]) * 2 : OOB);
#pragma unroll
    for (int i = 0; i < B_I; ++i)
      dma16(rw_rsrc, sb + bdst[i],
            (k0 + bkc[i] < kend && boff[i] != OOB) ? boff[i] + (k0 + bkc[i]) * (W8 ? 1 : 2) : OOB);
  };

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // residual add: this lane's residual values are loaded now (the oldest loads in flight),
  // so the epilogue does not wait for them (wave tiles of up to 8 fragments: more would spill)
  constexpr bool PRE = EK == EPI_RESID_ADD && FM * FN <= 8 && !W8;  // (W8: the decode needs the registers)
  float4 res[PRE ? FM * FN : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = r0 + wm * TM + i * 16 + (lane & 15);
        const int n = n0 + wn * TN + j * 16 + (lane >> 4) * 4;
        res[i * FN + j] = (r < a.rows && n < a.N)
                              ? *(const float4*)((const float*)e.out + ((long)g * e.out_gstride + e.out_row_off + r) * e.out_ld + n)
                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    asm volatile("" ::: "memory");
  }

  // Fragment reads: row (wm*TM + i*16 + lane%16) of A, k-chunk ks*4 + lane/16; the row's
  // swizzle term depends on lane%16 only (fragment rows start at multiples of 16), so a
  // lane's element offset inside the fragment's 16 rows is fixed: fpos[ks].
  int fpos[BK / 32];
  if constexpr (BK == 32) {
    const int L = lane & 7, h = ((lane >> 3) & 1) | ((lane >> 4) << 1);
    fpos[0] = (L * 8 + (h ^ L)) * 8;
  } else {
    const int fsw = kswz64(lane & 15);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) fpos[ks] = (lane & 15) * BK + ((ks * 4 + (lane >> 4)) ^ fsw) * 8;
  }
  // e4m3 fragment reads: lane holds k = 32 ks + 8 (lane / 16) .. +7 of row lane % 16
  int fpos8[BK / 32];
#pragma unroll
  for (int ks = 0; ks < BK / 32; ++ks) {
    const int r16 = lane & 15, g = lane >> 4, c = (32 * ks + 8 * g) / 16;
    fpos8[ks] = r16 * BK + ((c ^ wswz8<CW>(r16)) * 16) + (g & 1) * 8;
  }
  auto compute = [&](auto st) {
    const uint16_t* sa = stage_a(st);
    const uint16_t* sb = stage_b(st);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int pos = fpos[ks];
      bf16x8_t af[FM], wf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const bf16x8_t*)&sa[(wm * TM + i * 16) * BK + pos];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (W8)
          wf[j] = e4m3x8_to_bf16x8(*(const uint2*)((const uint8_t*)sb + (wn * TN + j * 16) * BK + fpos8[ks]));
        else
          wf[j] = *(const bf16x8_t*)&sb[(wn * TN + j * 16) * BK + pos];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[j], af[i], acc[i][j], 0, 0, 0);
    }
  };
  // Step kt (stage kt % ST): wait for its loads (the ST - 2 later stages stay in flight)
  // and for every wave to be done with the stage read in the previous step, refill that
  // stage with k-tile kt + ST - 1, multiply.
  auto step = [&](auto st, int kt) {
    wait_vm_barrier<PER_STAGE * (ST - 2)>();
    issue(ic<(decltype(st)::value + ST - 1) % ST>{}, kt + ST - 1);
    compute(st);
  };

  const int nk = (kend - kbeg + BK - 1) / BK;
  for_seq<ST - 1>([&](auto i) { issue(i, decltype(i)::value); });
  int kt = 0;
  for (; kt + ST <= nk; kt += ST) for_seq<ST>([&](auto i) { step(i, kt + decltype(i)::value); });
  for_seq<ST - 1>([&](auto i) {
    if (kt + decltype(i)::value < nk) step(i, kt + decltype(i)::value);
  });
  // no load may still be writing LDS when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  mfma_epilogue<BM, BN, WM, WN, EK>(a, e, acc, g, cat, split, r0, n0, wm, wn, lane, PRE ? res : nullptr, bfirst,
                                    brows);
}

// ------------------------------------------------------------------------------------
// W8A8: e4m3 activations x e4m3 weights on the gfx950 fp8 matrix instruction
// (v_mfma_f32_16x16x128_f8f6f4, both operands e4m3, no block scales). Both operands are
// byte rows, A [rows][K] (row stride lda bytes) and W [N][K]; one stage holds 128 k of each,
// i.e. 128-byte rows laid out in LDS as the bf16 kernel's 64-deep tiles (chunk c of row r at
// position c ^ kswz64(r)), loaded by the same direct-to-LDS ring. A fragment (lane l: row
// l % 16, k = 32 (l / 16) .. +31, 32 bytes) is two 16-byte LDS reads. Products accumulate in
// fp32 (k-tiles in order, 128 k per instruction); each accumulator row is then multiplied by
// its activation scale (a.ascale[row]) and the epilogue applies the weight column scales.
// ------------------------------------------------------------------------------------
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int BM, int BN, int WM, int WN, int ST, int EK, int GM>
__global__ __launch_bounds__(64 * WM * WN) void gemm_a8_kernel(GemmArgs a, Epi e) {
  constexpr int BK = 128;            // k (= bytes) of one stage row
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int RPI = 8;             // tile rows per wave load instruction (8 chunks per row)
  constexpr int A_I = BM / (RPI * NW), B_I = BN / (RPI * NW);
  static_assert(A_I >= 1 && B_I >= 1 && A_I * RPI * NW == BM && B_I * RPI * NW == BN,
                "tile rows must split evenly over the waves");
  static_assert(FM >= 1 && FN >= 1, "tile shape");
  static_assert(ST >= 2 && ST <= 4, "2 to 4 stages");
  constexpr int PER_STAGE = A_I + B_I;
  static_assert(PER_STAGE * (ST - 1) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t As0[BM * BK], As1[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t As2[ST > 2 ? BM * BK : 16], As3[ST > 3 ? BM * BK : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs0[BN * BK], Bs1[BN * BK];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs2[ST > 2 ? BN * BK : 16], Bs3[ST > 3 ? BN * BK : 16];
  auto stage_a = [&](auto st) -> uint8_t* {
    constexpr int V = decltype(st)::value;
    if constexpr (V == 0) return As0;
    else if constexpr (V == 1) return As1;
    else if constexpr (V == 2) return As2;
    else return As3;
  };
  auto stage_b = [&](auto st) -> uint8_t* {
    constexpr int V = decltype(st)::value;
    if constexpr (V == 0) return Bs0;
    else if constexpr (V == 1) return Bs1;
    else if constexpr (V == 2) return Bs2;
    else return Bs3;
  };

  if (a.rows_dev) {
    a.rows = min(a.rows, *a.rows_dev);
    if ((int)blockIdx.x >= ((a.rows + BM - 1) / BM) * ((a.N + BN - 1) / BN)) return;
  }
  const int nm = (a.rows + BM - 1) / BM, nn = (a.N + BN - 1) / BN;
  int tm, tn, split;
  if (gridDim.z > 1 && gridDim.y == 1 && (8 % gridDim.z) == 0 && ((nm * nn * (int)gridDim.z) & 7) == 0) {
    split_tile_of<GM>(nm, nn, (int)gridDim.z, tm, tn, split);
  } else {
    tile_of<GM>(nm, nn, tm, tn);
    split = blockIdx.z;
  }
  const int r0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * a.k_per_split;
  const int kend = min(a.K, kbeg + a.k_per_split);
  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(a.A, (uint32_t)((long)a.rows * a.lda));
  const __amdgpu_buffer_rsrc_t rw_rsrc = make_rsrc(a.W, (uint32_t)((long)a.N * a.K));

  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave / WN, wn = wave % WN;

  // load instruction i of this wave fills LDS chunks 64 (wave * X_I + i) .. +63; lane l writes
  // row l / 8 of that block at chunk position l % 8, which holds k-chunk (l % 8) ^ kswz64(row)
  int aoff[A_I], akc[A_I], boff[B_I], bkc[B_I];
#pragma unroll
  for (int i = 0; i < A_I; ++i) {
    const int row = (wave * A_I + i) * RPI + (lane >> 3);
    aoff[i] = (r0 + row < a.rows) ? (r0 + row) * (int)a.lda : OOB;
    akc[i] = ((lane & 7) ^ kswz64(row & 15)) * 16;
  }
#pragma unroll
  for (int i = 0; i < B_I; ++i) {
    const int row = (wave * B_I + i) * RPI + (lane >> 3);
    boff[i] = (n0 + row < a.N) ? (n0 + row) * a.K : OOB;
    bkc[i] = ((lane & 7) ^ kswz64(row & 15)) * 16;
  }
  // every step issues its loads, also past the last k-tile (out of range: zeros, no traffic)
  auto issue = [&](auto st, int kt) {
    uint8_t* sa = stage_a(st);
    uint8_t* sb = stage_b(st);
    const int k0 = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < A_I; ++i)
      dma16(ra_rsrc, (uint16_t*)(sa + (wave * A_I + i) * 1024),
            (k0 + akc[i] < kend && aoff[i] != OOB) ? aoff[i] + k0 + akc[i] : OOB);
#pragma unroll
    for (int i = 0; i < B_I; ++i)
      dma16(rw_rsrc, (uint16_t*)(sb + (wave * B_I + i) * 1024),
            (k0 + bkc[i] < kend && boff[i] != OOB) ? boff[i] + k0 + bkc[i] : OOB);
  };

  floatx4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // fragment reads: row lane % 16 of the fragment, k-chunks 2 (lane / 16) and 2 (lane / 16) + 1
  const int fsw = kswz64(lane & 15);
  const int fp0 = (lane & 15) * BK + (((lane >> 4) * 2) ^ fsw) * 16;
  const int fp1 = (lane & 15) * BK + (((lane >> 4) * 2 + 1) ^ fsw) * 16;
  auto frag = [&](const uint8_t* base) -> i32x8_t {
    const i32x4_t lo = *(const i32x4_t*)(base + fp0);
    const i32x4_t hi = *(const i32x4_t*)(base + fp1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto compute = [&](auto st) {
    const uint8_t* sa = stage_a(st);
    const uint8_t* sb = stage_b(st);
    i32x8_t af[FM], wf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = frag(sa + (wm * TM + i * 16) * BK);
#pragma unroll
    for (int j = 0; j < FN; ++j) wf[j] = frag(sb + (wn * TN + j * 16) * BK);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], af[i], acc[i][j], 0, 0, 0, 0, 0, 0);
  };
  auto step = [&](auto st, int kt) {
    wait_vm_barrier<PER_STAGE * (ST - 2)>();
    issue(ic<(decltype(st)::value + ST - 1) % ST>{}, kt + ST - 1);
    compute(st);
  };

  const int nk = (kend - kbeg + BK - 1) / BK;
  for_seq<ST - 1>([&](auto i) { issue(i, decltype(i)::value); });
  int kt = 0;
  for (; kt + ST <= nk; kt += ST) for_seq<ST>([&](auto i) { step(i, kt + decltype(i)::value); });
  for_seq<ST - 1>([&](auto i) {
    if (kt + decltype(i)::value < nk) step(i, kt + decltype(i)::value);
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // activation row scales (rows past the end keep 1: the epilogue skips them)
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = r0 + wm * TM + i * 16 + (lane & 15);
    const float sr = r < a.rows ? a.ascale[r] : 1.0f;
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] *= sr;
  }
  mfma_epilogue<BM, BN, WM, WN, EK>(a, e, acc, 0, 0, split, r0, n0, wm, wn, lane, nullptr);
}

// ------------------------------------------------------------------------------------
// Skinny MFMA GEMM for <= 64 rows per group (weight streaming: B = 1 projections and
// the per-embodiment linears). A workgroup owns 16 output columns; its NWAVE waves take
// contiguous slices of K. Each lane loads its weight fragments (16 B of one weight row)
// and activation fragments straight from memory, a chunk of KC k-steps at a time with
// all loads of the chunk issued before the MFMAs, so a wave keeps KC x 16 B of weights
// in flight. The waves' partial sums are added through LDS in wave order.
// ------------------------------------------------------------------------------------
template <int MF, int NWAVE, bool FP8, int EK>
__global__ __launch_bounds__(64 * NWAVE) void gemm_skinny_kernel(GemmArgs a, Epi e) {
  constexpr int KC = 8;
  __shared__ floatx4_t red[NWAVE][MF][64];
  const int g = blockIdx.y;
  const int split = blockIdx.z;
  const int cat = a.ids ? a.ids[g] : 0;
  const int n0 = blockIdx.x * 16;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, lg = lane >> 4, lr = lane & 15;
  const uint32_t wes = FP8 ? 1 : 2;
  const uint16_t* A = (const uint16_t*)a.A + ((long)g * a.a_gstride + a.a_row_off) * a.lda;
  const char* Wb = (const char*)a.W + (long)cat * a.w_cstride * wes;
  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(A, (uint32_t)((long)a.rows * a.lda * 2));
  const __amdgpu_buffer_rsrc_t rw_rsrc = make_rsrc(Wb, (uint32_t)((long)a.N * a.K * wes));
  // k-steps of 32 of this split ([kbeg, kend) is a multiple of 32 wide except at K's end)
  const int kbeg = split * a.k_per_split, kend = min(a.K, kbeg + a.k_per_split);
  const int nsteps = (kend - kbeg + 31) / 32;
  const int spw = (nsteps + NWAVE - 1) / NWAVE;
  const int s0 = wave * spw, s1 = min(nsteps, s0 + spw);
  const int woff = (n0 + lr < a.N) ? (n0 + lr) * a.K * (int)wes : OOB;
  int aoff[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) aoff[mf] = (mf * 16 + lr < a.rows) ? (mf * 16 + lr) * (int)a.lda * 2 : OOB;

  floatx4_t acc[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) acc[mf] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = s0; c0 < s1; c0 += KC) {
    uint4 wv[KC];
    uint4 av[KC][MF];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int k = kbeg + (c0 + i) * 32 + lg * 8;
      const bool in = (c0 + i) < s1 && k < kend;
      if (FP8) {
        int32x4_t raw = {0, 0, 0, 0};
        const int off = (in && woff != OOB) ? woff + k : OOB;
        const auto lo = __builtin_amdgcn_raw_buffer_load_b64(rw_rsrc, off, 0, 0);
        raw[0] = lo[0];
        raw[1] = lo[1];
        wv[i] = make_uint4((uint32_t)raw[0], (uint32_t)raw[1], 0, 0);
      } else {
        wv[i] = buf_load16(rw_rsrc, (in && woff != OOB) ? woff + k * 2 : OOB);
      }
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) av[i][mf] = buf_load16(ra_rsrc, (in && aoff[mf] != OOB) ? aoff[mf] + k * 2 : OOB);
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      uint4 w = wv[i];
      if (FP8)
        w = make_uint4(e4m3x2_to_bf16x2(wv[i].x), e4m3x2_to_bf16x2(wv[i].x >> 16), e4m3x2_to_bf16x2(wv[i].y),
                       e4m3x2_to_bf16x2(wv[i].y >> 16));
      const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, w);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
        acc[mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, __builtin_bit_cast(bf16x8_t, av[i][mf]), acc[mf], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) red[wave][mf][lane] = acc[mf];
  __syncthreads();
  if (t < MF * 64) {
    const int mf = t >> 6, ln = t & 63;
    floatx4_t sum = red[0][mf][ln];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) sum += red[w][mf][ln];
    const int r = mf * 16 + (ln & 15);
    const int n = n0 + 4 * (ln >> 4);
    if (r < a.rows && n < a.N) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sc = a.wscale ? a.wscale[(long)cat * a.s_cstride + n + q] : 1.0f;
        const float bi = (a.bias && (EK != EPI_PARTIAL || split == 0)) ? a.bias[(long)cat * a.b_cstride + n + q] : 0.0f;
        v[q] = sum[q] * sc + bi;
      }
      epi_store<EK, 4>(e, g, r, n, v, cat, split);
    }
  }
}

// Variant for bf16 weights whose activation rows of the split fit in LDS: every workgroup
// reads the same few rows, and fetching them per lane as 16-row fragments costs more
// than the weight stream itself. Instead the workgroup copies its rows into LDS once
// (coalesced loads straight into LDS, rows padded by 16 bytes so that the 16 rows of a
// fragment read fall on distinct bank groups), while each wave's weight loads for its
// whole slice of K (at most KC k-steps) are already in flight. LN: the rows are the fp32
// residual stream instead, normalised (GemmArgs::ln) by the waves as they stage them.
constexpr int SKL_MAX_LDS = 64 * 1024;
template <int MF, int NC, int NWAVE, int EK, int LNV = 0, int KCW = 8>
__global__ __launch_bounds__(64 * NWAVE) void gemm_skinny_lds_kernel(GemmArgs a, Epi e) {
  constexpr bool LN = LNV > 0;  // LN: the rows are K = 256 LNV fp32 values, normalised here
  // k-steps of 32 loaded per wave (at most): with the LayerNorm, 8 waves over K = 256 LNV
  constexpr int KC = LN ? LNV : KCW;
  extern __shared__ __attribute__((aligned(1024))) uint16_t skl[];
  const int g = blockIdx.y;
  const int split = blockIdx.z;
  const int cat = a.ids ? a.ids[g] : 0;
  const int n0 = blockIdx.x * 16 * NC;  // NC 16-column fragments per workgroup
  const int t = threadIdx.x, lane = t & 63, lg = lane >> 4, lr = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint16_t* A = (const uint16_t*)a.A + ((long)g * a.a_gstride + a.a_row_off) * a.lda;
  const uint16_t* W = (const uint16_t*)a.W + (long)cat * a.w_cstride;
  const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(A, (uint32_t)((long)a.rows * a.lda * 2));
  const __amdgpu_buffer_rsrc_t rw_rsrc = make_rsrc(W, (uint32_t)((long)a.N * a.K * 2));
  const int kbeg = split * a.k_per_split, kend = min(a.K, kbeg + a.k_per_split);
  const int kper = a.k_per_split;            // multiple of 128
  const int rs = kper + 8;                   // padded LDS row (elements)
  const int cpr = rs / 8;                    // 16-byte chunks per padded row
  const int tc = a.rows * cpr;               // chunks of the staged rows

  // 0. the bias of the outputs this thread writes in 4. (first, so its latency overlaps the rest)
  float4 bias4[(NC * MF * 64 + 64 * NWAVE - 1) / (64 * NWAVE)];
#pragma unroll
  for (int u = 0; u < (NC * MF * 64 + 64 * NWAVE - 1) / (64 * NWAVE); ++u) {
    const int p = t + u * 64 * NWAVE, f = p >> 6, n = n0 + (f / MF) * 16 + 4 * ((p & 63) >> 4);
    bias4[u] = (a.bias && (EK != EPI_PARTIAL || split == 0) && p < NC * MF * 64 && n < a.N)
                   ? *(const float4*)(a.bias + (long)cat * a.b_cstride + n)
                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  // 1. activation rows [0, rows) x [kbeg, kbeg + kper) -> LDS (chunk c: row c / cpr, k-chunk c % cpr;
  //    the padding chunk and k past kend read 0)
  constexpr int LR = (MF * 16 + NWAVE - 1) / NWAVE, LV = LN ? LNV : 1;  // LN: rows per wave, float4 per lane
  float4 xv[LN ? LR : 1][LV];
  if constexpr (LN) {
    // rows wave, wave + NWAVE, ... of the fp32 residual stream, whole rows (kper = K); the
    // registers of rows past a.rows are neither loaded nor read (every test below is uniform)
    const float* hr = (const float*)a.A + 4 * lane;
#pragma unroll
    for (int r = 0; r < LR; ++r) {
      const int row = wave + r * NWAVE;
      if (row < a.rows) {
#pragma unroll
        for (int i = 0; i < LV; ++i) xv[r][i] = *(const float4*)(hr + (long)row * a.lda + 256 * i);
      }
    }
    // every wave's row loads enter the CU's load queue before any weight load: the rows are
    // needed first (for the LayerNorm, while the weights stream). No wait for their data.
    asm volatile("s_barrier" ::: "memory");
  } else {
    for (int j = wave; j * 64 < tc; j += NWAVE) {
      const int c = j * 64 + lane;
      const int row = c / cpr, kc = c - row * cpr;
      const int k = kbeg + kc * 8;
      const bool in = c < tc && kc < cpr - 1 && k < kend;
      dma16(ra_rsrc, skl + j * 64 * 8, in ? (row * (int)a.lda + k) * 2 : OOB);
    }
  }
  // the weight loads below must be issued after these (the wait in 3. counts on it)
  asm volatile("" ::: "memory");
  // 2. this wave's weight fragments: k-steps [s0, s1) of 32 of the split, NC column fragments
  const int nsteps = (kend - kbeg + 31) / 32;
  const int spw = (nsteps + NWAVE - 1) / NWAVE;
  const int s0 = wave * spw, s1 = min(nsteps, s0 + spw);
  int woff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) woff[c] = (n0 + c * 16 + lr < a.N) ? (n0 + c * 16 + lr) * a.K * 2 : OOB;
  // (unconditional, so that the compiler's waits before the products stay per load; a load
  // at an out-of-range offset still takes its turn on the CU's load path, so the launcher
  // picks KC = the k-steps per wave where it can)
  uint4 wv[KC][NC];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int k = kbeg + (s0 + i) * 32 + lg * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      wv[i][c] = buf_load16(rw_rsrc, (s0 + i < s1 && k < kend && woff[c] != OOB) ? woff[c] + k * 2 : OOB);
  }
  if constexpr (LN) {
    // nothing below may be scheduled above the weight loads (the row sums would wait for them)
    __builtin_amdgcn_sched_barrier(0);
    // 1'. each row: the mean, then the mean squared deviation from it, over its K values (two
    //     passes; the reductions of the wave's rows interleaved), normalised, modulated, bf16
    //     into LDS
    const float inv_k = 1.0f / (float)a.K;
    float mean[LR], s2[LR];
#pragma unroll
    for (int r = 0; r < LR; ++r) {
      mean[r] = 0.0f;
      if (wave + r * NWAVE < a.rows) {
#pragma unroll
        for (int i = 0; i < LV; ++i) mean[r] += (xv[r][i].x + xv[r][i].y) + (xv[r][i].z + xv[r][i].w);
      }
    }
    wave_sum_n(mean);
#pragma unroll
    for (int r = 0; r < LR; ++r) {
      mean[r] *= inv_k;
      s2[r] = 0.0f;
      if (wave + r * NWAVE < a.rows) {
#pragma unroll
        for (int i = 0; i < LV; ++i) {
          const float d0 = xv[r][i].x - mean[r], d1 = xv[r][i].y - mean[r], d2 = xv[r][i].z - mean[r],
                      d3 = xv[r][i].w - mean[r];
          s2[r] += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
        }
      }
    }
    wave_sum_n(s2);
#pragma unroll
    for (int r = 0; r < LR; ++r) {
      const int row = wave + r * NWAVE;
      if (row >= a.rows) break;
      const float rstd = rsqrtf(s2[r] * inv_k + 1e-5f);
#pragma unroll
      for (int i = 0; i < LV; ++i) {
        const int c = 4 * lane + 256 * i;
        float o[4] = {(xv[r][i].x - mean[r]) * rstd, (xv[r][i].y - mean[r]) * rstd, (xv[r][i].z - mean[r]) * rstd,
                      (xv[r][i].w - mean[r]) * rstd};
        if (a.ln_ada) {
          const float4 sc = *(const float4*)(a.ln_ada + c);
          const float4 sh = *(const float4*)(a.ln_ada + a.K + c);
          o[0] = o[0] * (1.0f + sc.x) + sh.x;
          o[1] = o[1] * (1.0f + sc.y) + sh.y;
          o[2] = o[2] * (1.0f + sc.z) + sh.z;
          o[3] = o[3] * (1.0f + sc.w) + sh.w;
        }
        *(uint2*)&skl[row * rs + c] = make_uint2(bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3]));
      }
    }
    __syncthreads();  // 3. the staged rows are complete (weight loads may still be in flight)
  } else {
    wait_vm_barrier<KC * NC>();  // 3. the staged rows are complete (weight loads may still be in flight)
  }
  floatx4_t acc[NC][MF];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[c][mf] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    if (s0 + i < s1) {
      const int kk = (s0 + i) * 32 + lg * 8;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const int row = mf * 16 + lr;
        const uint4 av = *(const uint4*)&skl[min(row, a.rows - 1) * rs + kk];
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, row < a.rows ? av : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[c][mf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[i][c]), af, acc[c][mf], 0, 0, 0);
      }
    }
  }
  // 4. the waves' partial sums, added in wave order through LDS (reusing the staged rows)
  __syncthreads();
  floatx4_t* red = (floatx4_t*)skl;  // [NWAVE][NC * MF][64]
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) red[(wave * NC * MF + c * MF + mf) * 64 + lane] = acc[c][mf];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (NC * MF * 64 + 64 * NWAVE - 1) / (64 * NWAVE); ++u) {
    const int p = t + u * 64 * NWAVE;
    if (p >= NC * MF * 64) break;
    const int f = p >> 6, ln = p & 63;  // f = c * MF + mf
    floatx4_t sum = red[f * 64 + ln];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) sum += red[(w * NC * MF + f) * 64 + ln];
    const int r = (f % MF) * 16 + (ln & 15);
    const int n = n0 + (f / MF) * 16 + 4 * (ln >> 4);
    if (r < a.rows && n < a.N) {
      float v[4] = {sum[0] + bias4[u].x, sum[1] + bias4[u].y, sum[2] + bias4[u].z, sum[3] + bias4[u].w};
      epi_store<EK, 4>(e, g, r, n, v, cat, split);
    }
  }
}

// LDS bytes gemm_skinny_lds_kernel needs (0 = does not fit).
static size_t skinny_lds_bytes(const GemmArgs& a, int mf, int nc, int nwave) {
  const long tc = (long)a.rows * ((a.k_per_split + 8) / 8);
  const long bytes = std::max(((tc + 63) / 64) * 64 * 16, (long)nwave * nc * mf * 1024);
  return bytes <= SKL_MAX_LDS ? (size_t)bytes : 0;
}

template <int MF, int NC, int NWAVE, int KC>
static hipError_t skinny_lds_kind(const GemmArgs& a, const Epi& e, int splits, size_t lds, hipStream_t s) {
  dim3 grid((a.N + 16 * NC - 1) / (16 * NC), a.groups, splits), blk(64 * NWAVE);
#define GR00T_SKL_CASE(K) \
  case K: hipLaunchKernelGGL((gemm_skinny_lds_kernel<MF, NC, NWAVE, K, 0, KC>), grid, blk, lds, s, a, e); break;
  switch (e.kind) {
    GR00T_SKL_CASE(EPI_STORE)
    GR00T_SKL_CASE(EPI_RESID_ADD)
    GR00T_SKL_CASE(EPI_HEADS)
    GR00T_SKL_CASE(EPI_EULER)
    GR00T_SKL_CASE(EPI_PARTIAL)
    default: return hipErrorInvalidValue;
  }
#undef GR00T_SKL_CASE
  return hipGetLastError();
}

// LayerNorm folded in (the MLP-up projection at a few rows): plain stores only, K = 256 LNV.
template <int MF>
static hipError_t skinny_ln_kind(const GemmArgs& a, const Epi& e, size_t lds, hipStream_t s) {
  dim3 grid((a.N + 31) / 32, 1, 1), blk(512);
  if (e.kind != EPI_STORE) return hipErrorInvalidValue;
  switch (a.K / 256) {
    case 4: hipLaunchKernelGGL((gemm_skinny_lds_kernel<MF, 2, 8, EPI_STORE, 4>), grid, blk, lds, s, a, e); break;
    case 5: hipLaunchKernelGGL((gemm_skinny_lds_kernel<MF, 2, 8, EPI_STORE, 5>), grid, blk, lds, s, a, e); break;
    case 6: hipLaunchKernelGGL((gemm_skinny_lds_kernel<MF, 2, 8, EPI_STORE, 6>), grid, blk, lds, s, a, e); break;
    case 7: hipLaunchKernelGGL((gemm_skinny_lds_kernel<MF, 2, 8, EPI_STORE, 7>), grid, blk, lds, s, a, e); break;
    case 8: hipLaunchKernelGGL((gemm_skinny_lds_kernel<MF, 2, 8, EPI_STORE, 8>), grid, blk, lds, s, a, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MF, int NWAVE, bool FP8>
static hipError_t skinny_kind(const GemmArgs& a, const Epi& e, int splits, hipStream_t s) {
  dim3 grid((a.N + 15) / 16, a.groups, splits), blk(64 * NWAVE);
#define GR00T_SKINNY_CASE(K) \
  case K: hipLaunchKernelGGL((gemm_skinny_kernel<MF, NWAVE, FP8, K>), grid, blk, 0, s, a, e); break;
  switch (e.kind) {
    GR00T_SKINNY_CASE(EPI_STORE)
    GR00T_SKINNY_CASE(EPI_RESID_ADD)
    GR00T_SKINNY_CASE(EPI_HEADS)
    GR00T_SKINNY_CASE(EPI_EULER)
    GR00T_SKINNY_CASE(EPI_PARTIAL)
    default: return hipErrorInvalidValue;
  }
#undef GR00T_SKINNY_CASE
  return hipGetLastError();
}

// Compute units of the current device (one query per process).
static int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    return n;
  }();
  return cus;
}

// The bf16 skinny kernel with staged rows streams each weight once; what bounds it is the
// load path of the busiest CU: every workgroup reads its 16 nc weight columns over its split
// of K and, in addition, the whole activation rows of that split (the same for every
// workgroup), and a CU holds ceil(workgroups / CUs) of them. Bytes through that CU:
static long skinny_cu_bytes(int rows, int N, int kper, int groups, int splits, int nc) {
  const long wgs = (long)((N + 16 * nc - 1) / (16 * nc)) * groups * splits;
  return ((wgs + device_cus() - 1) / device_cus()) * 2l * kper * (16 * nc + rows);
}
// Column fragments per workgroup (1 or 3) for a launch of the staged-rows kernel, 0 if it
// does not fit: 3 where that moves at least 5% fewer bytes through the busiest CU.
static int skinny_lds_nc(const GemmArgs& a, int mf, int splits) {
  const int kper = a.k_per_split;
  if (kper % 128 != 0 || kper > 2048) return 0;
  const int nwave1 = kper >= 1024 ? 8 : 4;
  if (kper > nwave1 * 256 || !skinny_lds_bytes(a, mf, 1, nwave1)) return 0;
  if (mf <= 2 && skinny_lds_bytes(a, mf, 3, 8) &&
      skinny_cu_bytes(a.rows, a.N, kper, a.groups, splits, 3) * 20 <
          skinny_cu_bytes(a.rows, a.N, kper, a.groups, splits, 1) * 19)
    return 3;
  return 1;
}

template <int MF>
static hipError_t skinny_go(const GemmArgs& a, const Epi& e, bool fp8, int splits, hipStream_t s) {
  // KC k-steps of 32 per wave: 8 waves cover a split of up to 2048, 4 up to 1024; where the
  // k-steps divide evenly into 3 or 6 per wave of 8, exactly that many (no idle loads)
  const int nc = fp8 ? 0 : skinny_lds_nc(a, MF, splits);
  if (nc) {
    const int nwave = (a.k_per_split >= 1024 || nc > 1) ? 8 : 4;
    const size_t lds = skinny_lds_bytes(a, MF, nc, nwave);
    const int nsteps = a.k_per_split / 32;
    if (nc == 3)
      return nsteps == 24 ? skinny_lds_kind<MF, 3, 8, 3>(a, e, splits, lds, s) : skinny_lds_kind<MF, 3, 8, 8>(a, e, splits, lds, s);
    if (nwave == 8)
      return nsteps == 48 ? skinny_lds_kind<MF, 1, 8, 6>(a, e, splits, lds, s) : skinny_lds_kind<MF, 1, 8, 8>(a, e, splits, lds, s);
    return skinny_lds_kind<MF, 1, 4, 8>(a, e, splits, lds, s);
  }
  const int nwave = a.k_per_split >= 1024 ? 8 : 4;
  if (a.k_per_split >= 1024)
    return fp8 ? skinny_kind<MF, 8, true>(a, e, splits, s) : skinny_kind<MF, 8, false>(a, e, splits, s);
  return fp8 ? skinny_kind<MF, 4, true>(a, e, splits, s) : skinny_kind<MF, 4, false>(a, e, splits, s);
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------
template <typename TA, typename TW>
static hipError_t valu_go(const GemmArgs& a, const Epi& e, hipStream_t s) {
  // few rows, deep K: split K inside the workgroup (vector loads: K and lda multiples of 4)
  if (a.rows <= VS_ROWS && a.K >= 4 * VS_SLICES && a.K % 4 == 0 && a.lda % 4 == 0 &&
      ((uintptr_t)a.A % 16) == 0 && ((uintptr_t)a.W % 16) == 0 && (a.w_cstride % 4) == 0 && (a.a_gstride * a.lda) % 4 == 0 &&
      ((long)a.a_row_off * a.lda) % 4 == 0) {
    dim3 grid((a.N + VS_COLS - 1) / VS_COLS, 1, a.groups);
    switch (e.kind) {
      case EPI_STORE: hipLaunchKernelGGL((gemm_valu_skinny_kernel<TA, TW, EPI_STORE>), grid, dim3(256), 0, s, a, e); break;
      case EPI_RESID_ADD: hipLaunchKernelGGL((gemm_valu_skinny_kernel<TA, TW, EPI_RESID_ADD>), grid, dim3(256), 0, s, a, e); break;
      case EPI_HEADS: hipLaunchKernelGGL((gemm_valu_skinny_kernel<TA, TW, EPI_HEADS>), grid, dim3(256), 0, s, a, e); break;
      case EPI_EULER: hipLaunchKernelGGL((gemm_valu_skinny_kernel<TA, TW, EPI_EULER>), grid, dim3(256), 0, s, a, e); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  dim3 grid((a.N + 63) / 64, (a.rows + 63) / 64, a.groups);
  switch (e.kind) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_valu_kernel<TA, TW, EPI_STORE>), grid, dim3(256), 0, s, a, e); break;
    case EPI_RESID_ADD: hipLaunchKernelGGL((gemm_valu_kernel<TA, TW, EPI_RESID_ADD>), grid, dim3(256), 0, s, a, e); break;
    case EPI_HEADS: hipLaunchKernelGGL((gemm_valu_kernel<TA, TW, EPI_HEADS>), grid, dim3(256), 0, s, a, e); break;
    case EPI_EULER: hipLaunchKernelGGL((gemm_valu_kernel<TA, TW, EPI_EULER>), grid, dim3(256), 0, s, a, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_valu(const GemmArgs& a, const Epi& e, DType at, DType wt, hipStream_t s) {
  if (a.rows <= 0 || a.N <= 0 || a.groups <= 0) return hipSuccess;
  if (at == DT_F32 && wt == DT_F32) return valu_go<float, float>(a, e, s);
  if (at == DT_F32 && wt == DT_BF16) return valu_go<float, bf16>(a, e, s);
  if (at == DT_BF16 && wt == DT_BF16) return valu_go<bf16, bf16>(a, e, s);
  if (at == DT_BF16 && wt == DT_F32) return valu_go<bf16, float>(a, e, s);
  return hipErrorInvalidValue;
}

// Tile configurations of the matrix-core GEMMs (tile_choice; measured on the head's shapes):
//   0: 256 x 256 (bf16; e4m3 weights 256 x 128), 16 waves   (many tiles: VL K/V projection, B >= 256)
//   1: 256 x 128, 16 waves, 64 k per stage, 3 stages        (B ~ 64: MLP up and down, fused q,k,v)
//   2: 64 x 128, 4 waves                                    (few tiles)
//   5: 128 x 64, 8 waves, 4 stages                          (narrow outputs: q and o projections)
// (3 and 4 name the <= 32 and <= 16 row cases, which the skinny kernels serve.)
template <int BM, int BN, int WM, int WN, int BK, int ST, int GM, bool W8 = false>
static hipError_t dma_kind(const GemmArgs& a, const Epi& e, int splits, hipStream_t s) {
  const int nm = (a.rows + BM - 1) / BM, nn = (a.N + BN - 1) / BN;
  dim3 grid(nm * nn, a.groups, splits);
  dim3 blk(64 * WM * WN);
#define GR00T_DMA_CASE(K) \
  case K: hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, WM, WN, BK, ST, K, GM, W8>), grid, blk, 0, s, a, e); break;
  switch (e.kind) {
    GR00T_DMA_CASE(EPI_STORE)
    GR00T_DMA_CASE(EPI_RESID_ADD)
    GR00T_DMA_CASE(EPI_HEADS)
    GR00T_DMA_CASE(EPI_EULER)
    GR00T_DMA_CASE(EPI_PARTIAL)
    default: return hipErrorInvalidValue;
  }
#undef GR00T_DMA_CASE
  return hipGetLastError();
}

static int tile_choice(int rows, int N, int groups) {
  auto tiles = [&](int bm, int bn) { return (long)((rows + bm - 1) / bm) * ((N + bn - 1) / bn) * groups; };
  if (rows <= 16) return 4;
  if (rows <= 32) return 3;
  if (rows <= 64) return 2;
  if (tiles(256, 128) >= 512) return 0;
  if (tiles(256, 128) >= 160) return 1;
  if (N <= 2048) return 5;  // narrow outputs: 128 x 64 tiles, 8 waves
  return 2;
}

// Smallest split count that gives >= 240 workgroups (or leaves <= 512 k per split),
// else the largest valid one (at most 8, each split a multiple of 64 deep).
int gemm_mfma_splits(int rows, int N, int K, int groups, bool bf16w) {
  static const int bm[6] = {256, 256, 64, 32, 16, 128}, bn[6] = {128, 128, 128, 64, 64, 64};
  if (rows <= 32 && bf16w) {
    // staged-rows kernel: the split depth (and column fragments) with the fewest bytes
    // through the busiest CU; a deeper split must save more than 5% (each split is one more
    // partial for the next norm to add)
    GemmArgs a{};
    a.rows = rows;
    a.N = N;
    a.groups = groups;
    int best = 0;
    long best_b = 0;
    for (int s = 1; s <= 8; ++s) {
      if (K % (128 * s) != 0) continue;
      a.k_per_split = K / s;
      const int nc = skinny_lds_nc(a, rows <= 16 ? 1 : 2, s);
      if (!nc) continue;
      const long b = skinny_cu_bytes(rows, N, K / s, groups, s, nc);
      if (!best || b * 20 < best_b * 19) best = s, best_b = b;
    }
    if (best) return best;
  }
  if (rows <= 64) {
    // skinny kernel: 8 waves split K inside a workgroup, each holding one chunk of 8 k-steps
    // (256 deep) in flight; deeper K is split across workgroups
    int s = 1;
    while (K / s > 2048 && s < 8 && K % (64 * s * 2) == 0) s *= 2;
    if (K / s > 2048 && K % (64 * 3) == 0 && K / 3 <= 2048) s = 3;
    // few column blocks (narrow N): split deeper until >= 256 workgroups, keeping K / s >= 384
    while ((long)((N + 15) / 16) * groups * s < 256 && s < 8 && K % (128 * s * 2) == 0 && K / (s * 2) >= 384) s *= 2;
    return s;
  }
  // 256 x 128 tiles if some split depth of at least 1024 fills the chip with them
  const long t256 = (long)((rows + 255) / 256) * ((N + 127) / 128) * groups;
  for (int s = 1; s <= 8 && K / s >= 1024; ++s)
    if (K % (64 * s) == 0 && t256 * s >= 240) return s;
  int best = 1;
  for (int s = 1; s <= 8; ++s) {
    if (K % (64 * s) != 0) continue;
    best = s;
    const int c = tile_choice(rows, N, groups * s);
    const long t = (long)((rows + bm[c] - 1) / bm[c]) * ((N + bn[c] - 1) / bn[c]) * groups * s;
    // narrow 128 x 64 tiles: 216 tiles at 1088 rows fill the chip well enough that splitting
    // (and the partials the next norm must add) costs more than it gains
    if (t >= (c == 5 ? 200 : 240) || K / s <= 512) return s;
  }
  return best;
}

bool gemm_ln_fits(int rows, int K, DType wt) {
  if (rows < 1 || rows > 32 || wt != DT_BF16 || K < 1024 || K > 2048 || K % 256 != 0) return false;
  GemmArgs a{};
  a.rows = rows;
  a.k_per_split = K;
  return skinny_lds_bytes(a, rows <= 16 ? 1 : 2, 2, 8) != 0;
}

hipError_t launch_gemm_mfma(const GemmArgs& a_in, const Epi& e, DType wt, hipStream_t s) {
  GemmArgs a = a_in;
  if (a.rows <= 0 || a.N <= 0 || a.groups <= 0) return hipSuccess;
  const bool fp8 = (wt == DT_FP8);
  if (!fp8 && wt != DT_BF16) return hipErrorInvalidValue;
  if ((a.K % (fp8 ? 16 : 8)) != 0 || (a.lda % 8) != 0 || (a.N % 4) != 0) return hipErrorInvalidValue;
  int splits = 1;
  if (e.kind == EPI_PARTIAL) {
    splits = e.splits;
    if (splits < 1 || a.K % (64 * splits) != 0) return hipErrorInvalidValue;
  }
  a.k_per_split = a.K / splits;
  if ((long)a.rows * a.lda * 2 >= (1l << 31) || (long)a.N * a.K * 2 >= (1l << 31)) return hipErrorInvalidValue;
  if (a.ln) {  // LayerNorm of the fp32 A rows folded into the skinny kernel
    if (!gemm_ln_fits(a.rows, a.K, wt) || splits != 1 || a.groups != 1 || a.a_row_off != 0 || a.lda < a.K)
      return hipErrorInvalidValue;
    // 32 columns per workgroup: the rows held in registers allow one workgroup per CU, so
    // half as many workgroups fit the chip in one round
    const size_t lds = skinny_lds_bytes(a, a.rows <= 16 ? 1 : 2, 2, 8);
    return a.rows <= 16 ? skinny_ln_kind<1>(a, e, lds, s) : skinny_ln_kind<2>(a, e, lds, s);
  }
  if (a.chunks) {
    // category buckets: 128-row tiles, one chunk of at most chunk_cap samples of `rows` rows
    // each per tile row; stores and the Euler update only, one split
    if (fp8 || a.ln || splits != 1 || a.rows_dev || (e.kind != EPI_STORE && e.kind != EPI_EULER) ||
        a.chunk_cap < 1 || (long)a.chunk_cap * a.rows > 128 || a.perm == nullptr || a.map_bytes <= 0 ||
        a.map_bytes >= (1l << 31))
      return hipErrorInvalidValue;
    return dma_kind<128, 64, 4, 2, 64, 4, 16>(a, e, 1, s);
  }
  if (a.rows <= 64) {
    if (a.rows <= 16) return skinny_go<1>(a, e, fp8, splits, s);
    if (a.rows <= 32) return skinny_go<2>(a, e, fp8, splits, s);
    return skinny_go<4>(a, e, fp8, splits, s);
  }
  const int cfg = tile_choice(a.rows, a.N, a.groups * splits);
  if (!fp8) {  // bf16 weights: tiles straight into LDS through a 3-stage ring
    // 16 waves (4 per SIMD): measured 4-8% faster than 8 waves with 64 x 64 wave tiles
    if (cfg == 0) return dma_kind<256, 256, 4, 4, 32, 4, 8>(a, e, splits, s);
    if (cfg == 1) return dma_kind<256, 128, 4, 4, 64, 3, 8>(a, e, splits, s);
    if (cfg == 2) return dma_kind<64, 128, 2, 2, 64, 3, 16>(a, e, splits, s);
    // 128 x 64 tiles: 24 steps of 64 k with little work each; a fourth stage keeps three
    // tiles of loads in flight (measured 9% faster than three stages)
    if (cfg == 5) return dma_kind<128, 64, 4, 2, 64, 4, 16>(a, e, splits, s);
  } else {  // e4m3 weights: the same tiles, weight bytes into LDS, decoded per fragment
    // 256 x 128 also where bf16 takes 256 x 256: with the decode, 64 x 64 wave tiles exceed
    // the 128 registers of four waves per SIMD
    if (cfg == 0 || cfg == 1) return dma_kind<256, 128, 4, 4, 64, 3, 8, true>(a, e, splits, s);
    if (cfg == 2) return dma_kind<64, 128, 2, 2, 64, 3, 16, true>(a, e, splits, s);
    if (cfg == 5) return dma_kind<128, 64, 4, 2, 64, 4, 16, true>(a, e, splits, s);
  }
  return hipErrorInvalidValue;  // more than 64 rows always selects one of the tiles above
}

template <int BM, int BN, int WM, int WN, int ST, int GM>
static hipError_t a8_kind(const GemmArgs& a, const Epi& e, int splits, hipStream_t s) {
  const int nm = (a.rows + BM - 1) / BM, nn = (a.N + BN - 1) / BN;
  dim3 grid(nm * nn, 1, splits);
  dim3 blk(64 * WM * WN);
#define GR00T_A8_CASE(K) \
  case K: hipLaunchKernelGGL((gemm_a8_kernel<BM, BN, WM, WN, ST, K, GM>), grid, blk, 0, s, a, e); break;
  switch (e.kind) {
    GR00T_A8_CASE(EPI_STORE)
    GR00T_A8_CASE(EPI_RESID_ADD)
    GR00T_A8_CASE(EPI_HEADS)
    GR00T_A8_CASE(EPI_PARTIAL)
    default: return hipErrorInvalidValue;
  }
#undef GR00T_A8_CASE
  return hipGetLastError();
}

hipError_t launch_gemm_a8(const GemmArgs& a_in, const Epi& e, hipStream_t s) {
  GemmArgs a = a_in;
  if (a.rows <= 0 || a.N <= 0) return hipSuccess;
  if (a.groups != 1 || a.ids != nullptr || a.a_gstride != 0 || a.a_row_off != 0 || a.ln || a.ascale == nullptr)
    return hipErrorInvalidValue;
  if (a.K % 16 != 0 || a.lda % 16 != 0 || a.lda < a.K || a.N % 4 != 0) return hipErrorInvalidValue;
  if ((long)a.rows * a.lda >= (1l << 31) || (long)a.N * a.K >= (1l << 31)) return hipErrorInvalidValue;
  int splits = 1;
  if (e.kind == EPI_PARTIAL) {
    splits = e.splits;
    if (splits < 1 || a.K % (64 * splits) != 0) return hipErrorInvalidValue;
  }
  a.k_per_split = a.K / splits;
  const int cfg = tile_choice(a.rows, a.N, splits);
  if (cfg == 0 || cfg == 1) return a8_kind<256, 128, 4, 4, 3, 8>(a, e, splits, s);
  if (cfg == 5) return a8_kind<128, 64, 4, 2, 4, 16>(a, e, splits, s);
  return a8_kind<64, 128, 2, 2, 3, 16>(a, e, splits, s);
}

}  // namespace gr00t

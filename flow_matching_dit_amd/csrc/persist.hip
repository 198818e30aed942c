// Persistent kernel for the DiT blocks of one sample (B = 1): every block of one Euler step
// in a single launch of one workgroup per CU.
//
// At B = 1 each block is a chain of small dependent steps (adaLN, q/k/v projection,
// attention, o projection, LayerNorm, MLP up, MLP down) over 1 + H rows, so the time of a
// launch-per-step design is set by launch gaps and memory round trips, not by the 56 MB of
// weights a block streams ("Model architecture", Transformer block structure). Here the
// 256 workgroups stay resident for the whole step and synchronise among themselves:
//
//  * Work is split by XCD. A workgroup reads the XCD it runs on from the hardware and takes a
//    ticket from that XCD's counter: its local index li (the grid's 256 workgroups are dealt
//    round-robin over the 8 XCDs, 32 each, but the first one need not land on XCD 0). XCD x
//    owns heads 4x .. 4x+3 (192 attention columns) and MLP columns 768x .. 768x+767;
//    workgroup li of the XCD owns 6 q (k, v) columns, 24 MLP columns and 48 columns of the
//    residual stream.
//  * Steps whose inputs come from the same XCD synchronise through that XCD's L2 (plain
//    stores, an arrival counter, then an L1 invalidate before the reads); the two steps that
//    add contributions of every XCD into the residual stream (o projection and MLP down, each
//    XCD holding a partial sum over its heads / MLP columns) exchange them through memory
//    with device-coherent stores and loads (sc1) and a two-level arrival counter (XCD, then
//    device). Every XCD keeps its own copy of the residual stream h in its L2.
//  * The weights a workgroup needs for its next projections do not depend on activations:
//    the 7 compute waves request them into registers while a barrier waits (a step ahead of
//    their use). An eighth, control wave requests no weights and does the barriers' arrivals
//    and polls, so its polls never queue behind the weight stream.
//  * Every wait is bounded: a wait that exceeds its poll budget sets an abort word that ends
//    every workgroup's loop, and counts itself in a sticky error word the host reads.
//
// Per block: adaLN -> q/q,k,v [XCD sync] -> attention [XCD sync] -> o projection partial
// [device sync] -> residual [XCD sync] -> LayerNorm -> MLP up + GELU [XCD sync] -> MLP down
// partial [device sync] -> residual [XCD sync]. The arithmetic per step is that of the
// launch-per-step path (bf16 operands, fp32 accumulation, fp32 residual stream, fp32
// LayerNorm statistics and softmax, erf GELU).
#include <hip/hip_runtime.h>

#include "kcommon.h"
#include "kernels.h"

namespace gr00t {
namespace {

constexpr int PD = 1536, PF = 6144, PNH = 32, PHD = 48;
constexpr int NX = 8, NWG = 32, PG = NX * NWG;  // XCDs, workgroups per XCD, grid
constexpr int CW = PD / NWG;                    // 48 residual columns per workgroup
constexpr int AX = (PNH / NX) * PHD;            // 192 attention columns per XCD
constexpr int QW = AX / NWG;                    // 6 q (and k, v) columns per workgroup
constexpr int FX = PF / NX;                     // 768 MLP columns per XCD
constexpr int FW = FX / NWG;                    // 24 MLP columns per workgroup
constexpr int NWAVE = 7, NT = 64 * (NWAVE + 1);  // 7 compute waves and the control wave
constexpr int SMAX = 32;                        // rows (tokens) at most
constexpr int ROW = PD + 8;                     // staged bf16 row pitch (elements)
constexpr int RCH = 17;                         // LayerNorm rows per pass
constexpr int KQ = 7;                           // k-steps per wave, K = 1536 (48 k-steps of 32)
constexpr int KD = 4;                           // k-steps per wave, K = 768 (24 k-steps)
constexpr int WA = 2 * KQ, WBN = 3 * KD;        // weight fragments per lane: q / MLP up, o / MLP down
constexpr unsigned SPIN = 1u << 20;             // polls before a wait gives up (PersistArgs::spin = 0)

// control words, one 256-byte line each
enum : int {
  C_ABORT = 0,
  C_XBAR = 64,       // + 64 x: XCD barrier arrivals
  C_DEV = 64 * 9,    // device barrier: XCDs arrived
  C_XREL = 64 * 10,  // + 64 x: device barrier released for XCD x
  C_XARR = 64 * 18,  // + 64 x: device barrier arrivals within XCD x
  C_TICKET = 64 * 26, // + 64 x: workgroups that started on XCD x
  C_ERR = 64 * 34,   // timed-out waits and layout failures (sticky: not cleared between launches)
  C_RESET = 64 * 34, // words cleared before every launch
  C_WORDS = 64 * 35
};

__device__ __forceinline__ unsigned ld_ag(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_ag(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(N): at most N vector memory operations of this wave still outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
// drop this CU's L1 lines: data other CUs of the XCD wrote is then read from the XCD's L2
__device__ __forceinline__ void l1_invalidate() { asm volatile("buffer_inv sc0" ::: "memory"); }
// Phase timestamps (builds with GR00T_PHASE_TRACE only): s_memrealtime (100 MHz) at the phase
// boundaries k = 0 .. 15 of every block, in workgroups (XCD 0, ticket 0) and (XCD 7, ticket 31),
// to trace[(which * PTRACE_BLOCKS + block) * 16 + k]; each launch overwrites the last one's.
constexpr int PTRACE_BLOCKS = 64;
#ifdef GR00T_PHASE_TRACE
#define PTS(k)                                                                                          \
  do {                                                                                                  \
    if (threadIdx.x == 0 && l < PTRACE_BLOCKS && ((x == 0 && li == 0) || (x == NX - 1 && li == NWG - 1))) \
      a.trace[((x == NX - 1) * PTRACE_BLOCKS + l) * 16 + (k)] = __builtin_amdgcn_s_memrealtime();      \
  } while (0)
#else
#define PTS(k) \
  do {         \
  } while (0)
#endif

__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 0xFu; }

// device-coherent 16-byte load / store (sc1): the partial sums other XCDs exchange
__device__ __forceinline__ float4 ld_sc1(__amdgpu_buffer_rsrc_t r, int off) {
  const int32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
  return make_float4(__int_as_float(v[0]), __int_as_float(v[1]), __int_as_float(v[2]), __int_as_float(v[3]));
}
__device__ __forceinline__ void st_sc1(__amdgpu_buffer_rsrc_t r, int off, float4 f) {
  int32x4_t v;
  v[0] = __float_as_int(f.x);
  v[1] = __float_as_int(f.y);
  v[2] = __float_as_int(f.z);
  v[3] = __float_as_int(f.w);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16);
}

__device__ bool spin_ge(const unsigned* p, unsigned target, unsigned* ctl, unsigned spin) {
  for (unsigned i = 0; i < spin; ++i) {
    if ((int)(ld_ag(p) - target) >= 0) return true;
    if ((i & 31u) == 31u && ld_ag(ctl + C_ABORT)) return false;
  }
  st_ag(ctl + C_ABORT, 1u);
  add_ag(ctl + C_ERR, 1u);
  return false;
}

// Barrier of the workgroups of XCD x (DEV = false) or of the whole grid (DEV = true). Every
// thread's global memory operations are complete before the control wave's first lane
// arrives; while it waits, the compute waves issue the weight requests `pre` for the steps
// ahead (the issue of a large request can stall a wave until the CU's share of memory
// bandwidth has taken it; here that stall overlaps the wait). After an XCD barrier the L1 is
// invalidated so that the reads that follow see the other workgroups' stores in L2.
template <bool DEV, typename Pre>
__device__ bool pbarrier(unsigned* ctl, int x, unsigned& n, int* sflag, unsigned spin, Pre&& pre) {
  const int wave = threadIdx.x >> 6;
  vm_wait<0>();
  __syncthreads();
  ++n;
  if (wave < NWAVE) {
    pre();
  } else if (threadIdx.x == 64 * NWAVE) {
    bool ok;
    if (DEV) {
      const unsigned old = add_ag(ctl + C_XARR + 64 * x, 1u);
      if (old + 1 == (unsigned)NWG * n) {  // last of the XCD: arrive for the XCD, then release it
        add_ag(ctl + C_DEV, 1u);
        ok = spin_ge(ctl + C_DEV, (unsigned)NX * n, ctl, spin);
        if (ok) st_ag(ctl + C_XREL + 64 * x, n);
      } else {
        ok = spin_ge(ctl + C_XREL + 64 * x, n, ctl, spin);
      }
    } else {
      add_ag(ctl + C_XBAR + 64 * x, 1u);
      ok = spin_ge(ctl + C_XBAR + 64 * x, (unsigned)NWG * n, ctl, spin);
    }
    *sflag = ok ? 1 : 0;
  }
  __syncthreads();
  if (!DEV) l1_invalidate();
  return __builtin_amdgcn_readfirstlane(*sflag) != 0;  // uniform: the loop stays scalar
}
template <bool DEV>
__device__ bool pbarrier(unsigned* ctl, int x, unsigned& n, int* sflag, unsigned spin) {
  return pbarrier<DEV>(ctl, x, n, sflag, spin, [] {});
}

// ------------------------------------------------------------------ weight fragments
// Weights are read once per step: non-temporal loads (nt), so that they do not evict the
// activations the XCD's workgroups exchange through L2.
__device__ __forceinline__ uint4 wload(__amdgpu_buffer_rsrc_t r, int off) {
  const int32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}
// The MFMA (v_mfma_f32_16x16x32_bf16) takes the weights as its first operand: lane l holds
// row (output column) 16 t + l % 16 of tile t and k = k0 + 8 (l / 16) .. +7, 16 bytes of the
// [out][in] packed matrix. Rows past the workgroup's columns read 0 (out-of-range offset).
__device__ __forceinline__ bf16x8_t bf(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// The requests of a projection are issued in slices of k-steps [S0, S1), spread over several
// barriers so that each barrier's share of the weight stream fits in its wait.

// q / q,k,v: self blocks 18 rows (q, k, v x 6 columns), cross blocks 6; wave w takes k-steps
// 7 w .. 7 w + 6 of the 48 (k = 32 ks + 8 (l / 16)). wb[t * KQ + s].
template <int S0, int S1>
__device__ __forceinline__ void load_wq(uint4 (&wb)[WA], const uint16_t* W, bool self, int x, int li, int wave,
                                        int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, (uint32_t)((self ? 3 : 1) * PD * PD * 2));
  const int nrows = self ? 3 * QW : QW;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 16 * t + lr;
    const int row = (r / QW) * PD + AX * x + QW * li + r % QW;
    const int base = r < nrows ? row * PD * 2 : OOB;
#pragma unroll
    for (int s = S0; s < S1; ++s) {
      const int ks = KQ * wave + s;
      wb[t * KQ + s] = wload(rs, (base == OOB || ks >= PD / 32) ? OOB : base + (32 * ks + 8 * lg) * 2);
    }
  }
}
// o projection: rows 48 li + 16 t + l % 16 (t < 3) of Wo [D][D], k = 192 x + 32 w + 8 (l / 16)
// (waves 0..5; one k-step each). wb[t].
__device__ __forceinline__ void load_wo(uint4 (&wb)[WBN], const uint16_t* W, int x, int li, int wave, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, (uint32_t)(PD * PD * 2));
#pragma unroll
  for (int t = 0; t < 3; ++t)
    wb[t] = wload(rs, wave < 6 ? ((CW * li + 16 * t + lr) * PD + AX * x + 32 * wave + 8 * lg) * 2 : OOB);
}
// MLP up: rows 768 x + 24 li + r (r < 24) of W1 [F][D]; k-steps as load_wq. wb[t * KQ + s].
template <int S0, int S1>
__device__ __forceinline__ void load_w1(uint4 (&wb)[WA], const uint16_t* W, int x, int li, int wave, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, (uint32_t)(PF * PD * 2));
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 16 * t + lr;
    const int base = r < FW ? (FX * x + FW * li + r) * PD * 2 : OOB;
#pragma unroll
    for (int s = S0; s < S1; ++s) {
      const int ks = KQ * wave + s;
      wb[t * KQ + s] = wload(rs, (base == OOB || ks >= PD / 32) ? OOB : base + (32 * ks + 8 * lg) * 2);
    }
  }
}
// MLP down: rows 48 li + 16 t + l % 16 of W2 [D][F]; k-steps w, w + 7, w + 14, w + 21 (< 24) of the
// XCD's 768 columns: k = 768 x + 32 ks + 8 (l / 16). wb[t * KD + s].
template <int S0, int S1>
__device__ __forceinline__ void load_w2(uint4 (&wb)[WBN], const uint16_t* W, int x, int li, int wave, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(W, (uint32_t)(PD * PF * 2));
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int s = S0; s < S1; ++s) {
      const int ks = wave + NWAVE * s;
      wb[t * KD + s] = wload(rs, ks < FX / 32 ? ((CW * li + 16 * t + lr) * PF + FX * x + 32 * ks + 8 * lg) * 2 : OOB);
    }
}

// A pointer every lane holds, moved to scalar registers (buffer descriptors built from it are
// then uniform; the block table is read with vector loads since the kernel writes global memory).
template <typename T>
__device__ __forceinline__ T* uniform(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ PBlock uniform_block(const PBlock* tab, int l) {
  const PBlock b = tab[l];
  PBlock u;
  u.wq = uniform(b.wq);
  u.bq = uniform(b.bq);
  u.wo = uniform(b.wo);
  u.bo = uniform(b.bo);
  u.w1 = uniform(b.w1);
  u.b1 = uniform(b.b1);
  u.w2 = uniform(b.w2);
  u.b2 = uniform(b.b2);
  u.nq = __builtin_amdgcn_readfirstlane(b.nq);
  return u;
}

// The value, opaque to the compiler: per-lane indices derived from it inside the block loop are
// recomputed where they are used instead of being kept live (in registers or spilled) across
// every step of the loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// ------------------------------------------------------------------ LayerNorm into LDS
// Row statistics come in two levels. Each workgroup, after updating its 48 columns of a row,
// stores their mean m_w and centred sum of squares M_w (publish_h); the LayerNorm combines
// the 32 partials of a row exactly (Chan et al.'s pairwise update with
// equal counts): mean = sum_w m_w / 32, M = sum_w M_w + 48 sum_w (m_w - mean)^2, var = M / D.

// Rows [0, S) of this XCD's copy of h, normalised with the combined statistics (eps 1e-5),
// times (1 + scale) plus shift when ada = [scale | shift] is given, rounded to bf16 into the
// staged rows. Thread t < 384 owns columns 4 t .. 4 t + 3; the 16 lanes of group t / 16 (< S)
// combine row t / 16's partials (two each). The rows, partials and modulation are requested
// together: one round trip to L2.
__device__ void ln_rows(const float* hx, const float2* stat /* [NWG][SMAX] of this XCD */, const float* ada, int S,
                        uint16_t* nl, float2* rs /* LDS [SMAX] */, int t) {
  const int c = 4 * t;
  const bool act = t < PD / 4;
  float4 xv[RCH];
#pragma unroll
  for (int i = 0; i < RCH; ++i)
    xv[i] = (act && i < S) ? *(const float4*)(hx + (long)i * PD + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 sc = make_float4(0.f, 0.f, 0.f, 0.f), sh = sc;
  if (ada && act) {
    sc = *(const float4*)(ada + c);
    sh = *(const float4*)(ada + PD + c);
  }
  const int srow = t >> 4, sw = 2 * (t & 15);
  float2 p0 = make_float2(0.f, 0.f), p1 = p0;
  if (srow < S) {
    p0 = stat[sw * SMAX + srow];
    p1 = stat[(sw + 1) * SMAX + srow];
  }
  if (t < 16 * S) {
    float sm = p0.x + p1.x;
    sm = row16_sum(sm);
    const float mean = sm / (float)NWG;
    const float d0 = p0.x - mean, d1 = p1.x - mean;
    float M = (p0.y + p1.y) + (float)CW * (d0 * d0 + d1 * d1);
    M = row16_sum(M);
    if ((t & 15) == 0) rs[srow] = make_float2(mean, 1.0f / sqrtf(M / (float)PD + 1e-5f));
  }
  __syncthreads();
  for (int r0 = 0; r0 < S; r0 += RCH) {
    if (r0 > 0) {
#pragma unroll
      for (int i = 0; i < RCH; ++i)
        xv[i] = (act && r0 + i < S) ? *(const float4*)(hx + (long)(r0 + i) * PD + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      if (!act || r0 + i >= S) continue;
      const float2 st = rs[r0 + i];
      float o[4] = {(xv[i].x - st.x) * st.y, (xv[i].y - st.x) * st.y, (xv[i].z - st.x) * st.y,
                    (xv[i].w - st.x) * st.y};
      if (ada) {
        o[0] = o[0] * (1.0f + sc.x) + sh.x;
        o[1] = o[1] * (1.0f + sc.y) + sh.y;
        o[2] = o[2] * (1.0f + sc.z) + sh.z;
        o[3] = o[3] * (1.0f + sc.w) + sh.w;
      }
      *(uint2*)&nl[(r0 + i) * ROW + c] = make_uint2(bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3]));
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ MFMA and the wave reduction

// acc[t][tt] += W fragment (tile t) x staged rows (token tile tt) over this wave's k-steps
// KQ * wave .. KQ * wave + KQ - 1 (those below 48)
template <int NTILE>
__device__ __forceinline__ void mma_lds(const uint4 (&wb)[WA], const uint16_t* nl, int S, int wave, int lane,
                                        floatx4_t (&acc)[3][2]) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < KQ; ++s) {
    if (KQ * wave + s >= PD / 32) break;
    asm volatile("" ::: "memory");  // keeps each k-step's LDS reads next to its MFMAs
    const int kk = 32 * (KQ * wave + s) + 8 * lg;
    const bf16x8_t b0 = bf(lr < S ? *(const uint4*)&nl[lr * ROW + kk] : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int t = 0; t < NTILE; ++t) acc[t][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(wb[t * KQ + s]), b0, acc[t][0], 0, 0, 0);
    if (S > 16) {
      const bf16x8_t b1 = bf(16 + lr < S ? *(const uint4*)&nl[(16 + lr) * ROW + kk] : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int t = 0; t < NTILE; ++t)
        acc[t][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(wb[t * KQ + s]), b1, acc[t][1], 0, 0, 0);
    }
  }
}

// Sum of the 7 compute waves' accumulators, in wave order, through LDS (red: 7 * 3 * 2 * 64 floatx4).
// Thread p < NTILE * 2 * 64 gets (t, tt, lane) = (p / 128, (p / 64) % 2, p % 64); returns false
// for the others.
template <int NTILE>
__device__ __forceinline__ bool wave_reduce(floatx4_t (&acc)[3][2], floatx4_t* red, int t, floatx4_t& sum, int& ti,
                                            int& tt, int& ln) {
  const int wave = t >> 6, lane = t & 63;
  __syncthreads();  // the staged rows under red are no longer read
  if (wave < NWAVE) {
#pragma unroll
    for (int a = 0; a < NTILE; ++a) {
      red[((wave * 3 + a) * 2 + 0) * 64 + lane] = acc[a][0];
      red[((wave * 3 + a) * 2 + 1) * 64 + lane] = acc[a][1];
    }
  }
  __syncthreads();
  if (t >= NTILE * 128) return false;
  ti = t >> 7;
  tt = (t >> 6) & 1;
  ln = t & 63;
  sum = red[((0 * 3 + ti) * 2 + tt) * 64 + ln];
#pragma unroll
  for (int w = 1; w < NWAVE; ++w) sum += red[((w * 3 + ti) * 2 + tt) * 64 + ln];
  return true;
}

__device__ __forceinline__ void zero_acc(floatx4_t (&acc)[3][2]) {
#pragma unroll
  for (int a = 0; a < 3; ++a) acc[a][0] = acc[a][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------ attention of one head

// The queries j0, j0 + 8, j0 + 16, j0 + 24 (< S) of head hl of this XCD, over Lk keys:
// self blocks the S rows of k / v in the XCD's q,k,v buffer, cross blocks the VL key / value
// caches with the key mask. softmax(q k^T / sqrt(hd)) v in fp32; a query with no admitted key
// outputs 0. The result rows go to the XCD's attention-output buffer (bf16, [SMAX][192]).
// Keys are taken in chunks of 32; thread j scores key j, thread (d, c) = (t % 48, t / 48) sums
// column d of value chunk c. The query, the first 512 key rows and the first 10 value chunks
// are requested together.
constexpr int PV_CH = NT / PHD;  // value chunks summed at once (10)

__device__ void attention_head(const PersistArgs& a, bool self, int cross_idx, int mask_bit, int x, int li, int t,
                               float* sm) {
  const int S = a.S, hl = li / 8, j0 = li % 8, head = (PNH / NX) * x + hl;
  const int nq = (S - j0 + 7) / 8 < 4 ? (S - j0 + 7) / 8 : 4;
  const uint16_t* qx = a.qkvx + (size_t)((x * 3 + 0) * (PNH / NX) + hl) * SMAX * PHD;
  const int Lk = self ? S : a.L;
  const int LKP = (Lk + 31) & ~31, nch = LKP / 32;
  // keys [Lk][hd] row-major (both kinds); values: self [S][hd] row-major, cross [Lp / 32][hd][32]
  const uint16_t* kb = self ? a.qkvx + (size_t)((x * 3 + 1) * (PNH / NX) + hl) * SMAX * PHD
                            : a.kc + cross_idx * a.kv_layer + (long)head * a.Lp * PHD;
  const uint16_t* vb = self ? a.qkvx + (size_t)((x * 3 + 2) * (PNH / NX) + hl) * SMAX * PHD
                            : a.vc + cross_idx * a.kv_layer + (long)head * a.Lp * PHD;
  float* qf = sm;               // [4][48], scaled by log2(e) / sqrt(hd)
  float* stat = sm + 4 * PHD;   // [4]: 1 / sum of the exponentials (0: no admitted key)
  float* p = stat + 4;          // [4][LKP] scores, then exponentials
  float* pvp = p + 4 * LKP;     // [PV_CH][4][48] partial outputs
  const float qscale = 1.4426950408889634f / sqrtf((float)PHD);
  // 1. requests: the query, key row t, value chunk t / 48 of column t % 48
  float qv = 0.f;
  if (t < nq * PHD) qv = bf16_to_f(qx[(j0 + 8 * (t / PHD)) * PHD + t % PHD]);
  auto key_admitted = [&](int j) { return j < Lk && (self || (a.code[j] & mask_bit) != 0); };
  auto load_key = [&](int j, uint4 (&kv)[PHD / 8]) {
#pragma unroll
    for (int c = 0; c < PHD / 8; ++c) kv[c] = *(const uint4*)(kb + (long)j * PHD + 8 * c);
  };
  auto load_val = [&](int c, int d, uint32_t (&vw)[16]) {  // keys 32 c .. 32 c + 31 of column d, bf16 pairs
    if (self) {
#pragma unroll
      for (int jj = 0; jj < 32; jj += 2) {
        const uint32_t lo = 32 * c + jj < S ? vb[(32 * c + jj) * PHD + d] : 0u;
        const uint32_t hi = 32 * c + jj + 1 < S ? vb[(32 * c + jj + 1) * PHD + d] : 0u;
        vw[jj / 2] = lo | (hi << 16);
      }
    } else {
      const uint4* v4 = (const uint4*)(vb + (long)c * PHD * 32 + d * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = v4[q];
        vw[4 * q] = u.x;
        vw[4 * q + 1] = u.y;
        vw[4 * q + 2] = u.z;
        vw[4 * q + 3] = u.w;
      }
    }
  };
  uint4 kv[PHD / 8];
  const bool kadm = key_admitted(t);
  if (kadm) load_key(t, kv);
  const int vd = t % PHD, vci = t / PHD;
  uint32_t vw[16];
  if (vci < PV_CH && vci < nch) load_val(vci, vd, vw);
  if (t < nq * PHD) qf[t] = qv * qscale;
  __syncthreads();
  // 2. scores (keys past Lk and masked keys: -inf)
  for (int jb = 0; jb < LKP; jb += NT) {
    const int j = jb + t;
    if (j >= LKP) break;
    const bool adm = jb == 0 ? kadm : key_admitted(j);
    if (jb > 0 && adm) load_key(j, kv);
    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
    if (adm) {
#pragma unroll
      for (int c = 0; c < PHD / 8; ++c) {
        const uint32_t w[4] = {kv[c].x, kv[c].y, kv[c].z, kv[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(w[e] << 16), k1 = __uint_as_float(w[e] & 0xFFFF0000u);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (m < nq) acc4[m] += qf[m * PHD + 8 * c + 2 * e] * k0 + qf[m * PHD + 8 * c + 2 * e + 1] * k1;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (m < nq) p[m * LKP + j] = adm ? acc4[m] : -INFINITY;
  }
  __syncthreads();
  // 3. softmax statistics: wave m for query m
  {
    const int wave = t >> 6, lane = t & 63;
    if (wave < nq) {
      float mx = -INFINITY;
      for (int j = lane; j < LKP; j += 64) mx = fmaxf(mx, p[wave * LKP + j]);
      mx = wave_max(mx);
      float sum = 0.f;
      for (int j = lane; j < LKP; j += 64) {
        const float e = mx == -INFINITY ? 0.f : exp2f(p[wave * LKP + j] - mx);
        p[wave * LKP + j] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) stat[wave] = sum > 0.f ? 1.0f / sum : 0.f;
    }
  }
  __syncthreads();
  // 4. p v: thread (vd, vci) sums chunks vci, vci + 10, ... of column vd
  if (vci < PV_CH) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = vci; c < nch; c += PV_CH) {
      if (c != vci) load_val(c, vd, vw);
#pragma unroll
      for (int jj = 0; jj < 32; jj += 2) {
        const float v0 = __uint_as_float(vw[jj / 2] << 16), v1 = __uint_as_float(vw[jj / 2] & 0xFFFF0000u);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (m < nq) acc[m] += p[m * LKP + 32 * c + jj] * v0 + p[m * LKP + 32 * c + jj + 1] * v1;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) pvp[(vci * 4 + m) * PHD + vd] = acc[m];
  }
  __syncthreads();
  if (t < nq * PHD) {
    const int m = t / PHD, d = t % PHD;
    float o = 0.f;
    for (int c = 0; c < PV_CH && c < nch; ++c) o += pvp[(c * 4 + m) * PHD + d];
    a.ox[((size_t)x * SMAX + j0 + 8 * m) * AX + hl * PHD + d] = f_to_bf16(o * stat[m]);
  }
}

// ------------------------------------------------------------------ the kernel

// The workgroup's 48 columns of h are held by 16-lane groups: thread t holds row t / 16,
// columns 48 li + 4 (t % 16) .. +3 when t % 16 < 12 (rows < S). They go to this XCD's copy of
// h, and their per-row partial statistics (mean m_w and centred sum of squares M_w of the 48
// values, a two-pass reduced across the row's 16 lanes) to stat_wg[row].
__device__ __forceinline__ void publish_h(float4 hs, bool hown, int hrow, int hcol, int t, int S, float* hx,
                                          float2* stat_wg) {
  if (hown) *(float4*)(hx + hrow * PD + hcol) = hs;
  if (t < 16 * S) {  // whole 16-lane groups: the shuffles below stay within a row
    float sm = hown ? (hs.x + hs.y) + (hs.z + hs.w) : 0.f;
    sm = row16_sum(sm);
    const float m = sm / (float)CW;
    const float d0 = hs.x - m, d1 = hs.y - m, d2 = hs.z - m, d3 = hs.w - m;
    float q = hown ? (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3) : 0.f;
    q = row16_sum(q);
    if ((t & 15) == 0) stat_wg[hrow] = make_float2(m, q);
  }
}

__global__ __launch_bounds__(NT) void dit_b1_persist_kernel(PersistArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int sflag;
  __shared__ float2 rstat[SMAX];
  uint16_t* nl = (uint16_t*)smem;     // staged rows [S][ROW] bf16
  floatx4_t* red = (floatx4_t*)smem;  // wave reduction (aliases the staged rows)
  float* asc = (float*)smem;          // attention scratch (aliases the staged rows)
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool cw = wave < NWAVE;       // compute wave (wave NWAVE: no weights; the barriers' polls)
  const int S = a.S;
  unsigned* ctl = a.ctl;
  const unsigned spin = a.spin ? a.spin : SPIN;
  unsigned nbx = 0, nbd = 0;
  __shared__ int sxl[2];
  if (t == 0) {
    const unsigned xc = xcc_id();
    const unsigned tk = xc < (unsigned)NX ? add_ag(ctl + C_TICKET + 64 * xc, 1u) : ~0u;
    sxl[0] = (int)xc;
    sxl[1] = (int)tk;
    sflag = (xc < (unsigned)NX && tk < (unsigned)NWG && gridDim.x == PG && S >= 1 && S <= SMAX) ? 1 : 0;
  }
  __syncthreads();
  const int x = __builtin_amdgcn_readfirstlane(sxl[0]), li = __builtin_amdgcn_readfirstlane(sxl[1]);
  if (!__builtin_amdgcn_readfirstlane(sflag)) {
    if (t == 0) {
      st_ag(ctl + C_ABORT, 1u);
      add_ag(ctl + C_ERR, 1u);
    }
    return;
  }
  // this workgroup's 48 columns of h (held as publish_h describes)
  float4 hs = ((t & 15) < 12 && t / 16 < S) ? *(const float4*)(a.h + (t / 16) * PD + CW * li + 4 * (t & 15))
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
  float* hx = a.hx + (size_t)x * SMAX * PD;  // this XCD's copy of h
  const float2* statx = a.statx + (size_t)x * NWG * SMAX;    // its rows' partial statistics
  float2* stat_wg = a.statx + ((size_t)x * NWG + li) * SMAX;  // this workgroup's
  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(a.part, (uint32_t)(2 * NX * SMAX * PD * 4));
  // two register sets of weight fragments: wa holds the q / q,k,v then the MLP up weights of a
  // block, wb the o projection then the MLP down weights
  uint4 wa[WA], wb[WBN];
  floatx4_t acc[3][2];
  publish_h(hs, (t & 15) < 12 && t / 16 < S, t / 16, CW * li + 4 * (t & 15), t, S, hx, stat_wg);
  bool ok = pbarrier<false>(ctl, x, nbx, &sflag, spin, [&] {
    const PBlock B0 = uniform_block(a.blocks, 0);
    load_wq<0, KQ>(wa, B0.wq, B0.nq == 3, x, li, wave, lane);
    load_wo(wb, B0.wo, x, li, wave, lane);
  });
  int par = 0, cross_idx = 0;
  for (int l = 0; l < a.nl && ok; ++l) {
    const PBlock B = uniform_block(a.blocks, l);
    const bool self = B.nq == 3;
    const bool more = l + 1 < a.nl;
    const int t = opaque(threadIdx.x), lane = t & 63, lr = lane & 15, lg = lane >> 4;
    const bool hown = (t & 15) < 12 && t / 16 < S;
    const int hrow = t / 16, hcol = CW * li + 4 * (t & 15);
    PTS(0);
    // ---- adaLN of h into the staged rows (block 0: the residual stream as the step starts)
    ln_rows(hx, statx, a.ada + (size_t)l * 2 * PD, S, nl, rstat, t);
    PTS(1);
    // ---- q (cross) or q, k, v (self) of this XCD's heads, the workgroup's 6 (18) columns
    zero_acc(acc);
    if (cw) mma_lds<2>(wa, nl, S, wave, lane, acc);
    {
      floatx4_t sum;
      int ti, tt, ln;
      if (wave_reduce<2>(acc, red, t, sum, ti, tt, ln)) {
        const int tok = 16 * tt + (ln & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ti + 4 * (ln >> 4) + i;
          if (tok < S && r < (self ? 3 : 1) * QW) {
            const int which = r / QW, col = QW * li + r % QW;  // column within the XCD's 192
            const float v = sum[i] + B.bq[which * PD + AX * x + col];
            a.qkvx[(((size_t)(x * 3 + which) * (PNH / NX) + col / PHD) * SMAX + tok) * PHD + col % PHD] = f_to_bf16(v);
          }
        }
      }
    }
    PTS(2);
    ok = pbarrier<false>(ctl, x, nbx, &sflag, spin, [&] { load_w1<0, 3>(wa, B.w1, x, li, wave, lane); });
    if (!ok) break;
    PTS(3);
    // ---- attention of one head for up to 4 queries
    attention_head(a, self, cross_idx, (l % (2 * a.text_every) == 0) ? 1 : 2, x, li, t, asc);
    PTS(4);
    ok = pbarrier<false>(ctl, x, nbx, &sflag, spin, [&] { load_w1<3, KQ>(wa, B.w1, x, li, wave, lane); });
    if (!ok) break;
    PTS(5);
    // ---- o projection: this XCD's partial sum over its 192 attention columns, for the
    //      workgroup's 48 output columns; then the MLP up and down weights are requested
    zero_acc(acc);
    if (cw && wave < 6) {
      const int kk = 32 * wave + 8 * lg;
      const uint16_t* ob = a.ox + (size_t)x * SMAX * AX;
      const bf16x8_t b0 = bf(lr < S ? *(const uint4*)&ob[lr * AX + kk] : make_uint4(0, 0, 0, 0));
      const bf16x8_t b1 = bf(16 + lr < S ? *(const uint4*)&ob[(16 + lr) * AX + kk] : make_uint4(0, 0, 0, 0));
#pragma unroll
      for (int ti = 0; ti < 3; ++ti) {
        acc[ti][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(wb[ti]), b0, acc[ti][0], 0, 0, 0);
        if (S > 16) acc[ti][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(wb[ti]), b1, acc[ti][1], 0, 0, 0);
      }
    }
    {
      floatx4_t sum;
      int ti, tt, ln;
      if (wave_reduce<3>(acc, red, t, sum, ti, tt, ln)) {
        const int tok = 16 * tt + (ln & 15), n = CW * li + 16 * ti + 4 * (ln >> 4);
        if (tok < S)
          st_sc1(rpart, (((par * NX + x) * SMAX + tok) * PD + n) * 4, make_float4(sum[0], sum[1], sum[2], sum[3]));
      }
    }
    PTS(6);
    ok = pbarrier<true>(ctl, x, nbd, &sflag, spin, [&] { load_w2<0, 2>(wb, B.w2, x, li, wave, lane); });
    if (!ok) break;
    PTS(7);
    // ---- residual: h += sum over the XCDs' partials (fixed order) + bo
    if (hown) {
      float4 p = ld_sc1(rpart, (((par * NX + 0) * SMAX + hrow) * PD + hcol) * 4);
#pragma unroll
      for (int y = 1; y < NX; ++y) {
        const float4 q = ld_sc1(rpart, (((par * NX + y) * SMAX + hrow) * PD + hcol) * 4);
        p.x += q.x;
        p.y += q.y;
        p.z += q.z;
        p.w += q.w;
      }
      const float4 bb = *(const float4*)(B.bo + hcol);
      hs.x += p.x + bb.x;
      hs.y += p.y + bb.y;
      hs.z += p.z + bb.z;
      hs.w += p.w + bb.w;
    }
    publish_h(hs, hown, hrow, hcol, t, S, hx, stat_wg);
    par ^= 1;
    PTS(8);
    ok = pbarrier<false>(ctl, x, nbx, &sflag, spin, [&] { load_w2<2, KD>(wb, B.w2, x, li, wave, lane); });
    if (!ok) break;
    PTS(9);
    // ---- LayerNorm, MLP up + GELU for the workgroup's 24 MLP columns
    ln_rows(hx, statx, nullptr, S, nl, rstat, t);
    PTS(10);
    zero_acc(acc);
    if (cw) mma_lds<2>(wa, nl, S, wave, lane, acc);
    {
      floatx4_t sum;
      int ti, tt, ln;
      if (wave_reduce<2>(acc, red, t, sum, ti, tt, ln)) {
        const int tok = 16 * tt + (ln & 15), r = 16 * ti + 4 * (ln >> 4);
        if (tok < S && r < FW) {
          const float4 bb = *(const float4*)(B.b1 + FX * x + FW * li + r);
          const float u0 = gelu_erf(sum[0] + bb.x), u1 = gelu_erf(sum[1] + bb.y), u2 = gelu_erf(sum[2] + bb.z),
                      u3 = gelu_erf(sum[3] + bb.w);
          *(uint2*)&a.ux[((size_t)x * SMAX + tok) * FX + FW * li + r] = make_uint2(bf16x2_bits(u0, u1), bf16x2_bits(u2, u3));
        }
      }
    }
    PTS(11);
    ok = pbarrier<false>(ctl, x, nbx, &sflag, spin, [&] {
      if (more) load_wq<0, 3>(wa, uniform(a.blocks[l + 1].wq), a.blocks[l + 1].nq == 3, x, li, wave, lane);
    });
    if (!ok) break;
    PTS(12);
    // ---- MLP down: this XCD's partial sum over its 768 MLP columns, for the workgroup's 48
    //      output columns; then the next block's q / q,k,v and o projection weights are requested
    zero_acc(acc);
    if (cw) {
      const uint16_t* ub = a.ux + (size_t)x * SMAX * FX;
#pragma unroll
      for (int s = 0; s < KD; ++s) {
        const int ks = wave + NWAVE * s;
        if (ks >= FX / 32) break;
        const int kk = 32 * ks + 8 * lg;
        const bf16x8_t b0 = bf(lr < S ? *(const uint4*)&ub[lr * FX + kk] : make_uint4(0, 0, 0, 0));
        const bf16x8_t b1 = bf(16 + lr < S ? *(const uint4*)&ub[(16 + lr) * FX + kk] : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int ti = 0; ti < 3; ++ti) {
          acc[ti][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(wb[ti * KD + s]), b0, acc[ti][0], 0, 0, 0);
          if (S > 16) acc[ti][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf(wb[ti * KD + s]), b1, acc[ti][1], 0, 0, 0);
        }
      }
    }
    {
      floatx4_t sum;
      int ti, tt, ln;
      if (wave_reduce<3>(acc, red, t, sum, ti, tt, ln)) {
        const int tok = 16 * tt + (ln & 15), n = CW * li + 16 * ti + 4 * (ln >> 4);
        if (tok < S)
          st_sc1(rpart, (((par * NX + x) * SMAX + tok) * PD + n) * 4, make_float4(sum[0], sum[1], sum[2], sum[3]));
      }
    }
    PTS(13);
    ok = pbarrier<true>(ctl, x, nbd, &sflag, spin, [&] {
      if (more) {
        const PBlock Bn = uniform_block(a.blocks, l + 1);
        load_wq<3, KQ>(wa, Bn.wq, Bn.nq == 3, x, li, wave, lane);
        load_wo(wb, Bn.wo, x, li, wave, lane);
      }
    });
    if (!ok) break;
    PTS(14);
    if (hown) {
      float4 p = ld_sc1(rpart, (((par * NX + 0) * SMAX + hrow) * PD + hcol) * 4);
#pragma unroll
      for (int y = 1; y < NX; ++y) {
        const float4 q = ld_sc1(rpart, (((par * NX + y) * SMAX + hrow) * PD + hcol) * 4);
        p.x += q.x;
        p.y += q.y;
        p.z += q.z;
        p.w += q.w;
      }
      const float4 bb = *(const float4*)(B.b2 + hcol);
      hs.x += p.x + bb.x;
      hs.y += p.y + bb.y;
      hs.z += p.z + bb.z;
      hs.w += p.w + bb.w;
    }
    if (more) publish_h(hs, hown, hrow, hcol, t, S, hx, stat_wg);
    par ^= 1;
    if (!self) ++cross_idx;
    if (more) ok = pbarrier<false>(ctl, x, nbx, &sflag, spin);
    PTS(15);
  }
  // the residual stream after the last block (every workgroup holds its 48 columns)
  if (ok && (t & 15) < 12 && t / 16 < S) *(float4*)(a.h + (t / 16) * PD + CW * li + 4 * (t & 15)) = hs;
}

__global__ void persist_reset_kernel(unsigned* ctl) {
  for (int i = threadIdx.x; i < C_RESET; i += blockDim.x) ctl[i] = 0u;
}

}  // namespace

size_t persist_lds_bytes(int S, int L) {
  const size_t rows = (size_t)S * ROW * 2;  // staged rows
  const size_t redb = (size_t)NWAVE * 3 * 2 * 64 * 16;
  const int lk = L > S ? L : S;
  const size_t attn = (size_t)(4 * PHD + 4 + 4 * ((lk + 31) & ~31) + PV_CH * 4 * PHD) * 4;
  size_t b = rows > redb ? rows : redb;
  if (attn > b) b = attn;
  // at least 96 KB: one workgroup per CU
  return b < 96 * 1024 ? 96 * 1024 : b;
}

bool persist_b1_fits(int D, int F, int nh, int hd, int S, int L, int num_devices_cus) {
  return D == PD && F == PF && nh == PNH && hd == PHD && S >= 1 && S <= SMAX && L >= 1 &&
         num_devices_cus == PG && persist_lds_bytes(S, L) <= 159 * 1024;
}

size_t persist_scratch_bytes() {
  return (size_t)NX * SMAX * PD * 4 +                        // hx
         (size_t)NX * 3 * (PNH / NX) * SMAX * PHD * 2 +      // qkvx
         (size_t)NX * SMAX * AX * 2 +                        // ox
         (size_t)NX * SMAX * FX * 2 +                        // ux
         (size_t)2 * NX * SMAX * PD * 4 +                    // part
         (size_t)NX * NWG * SMAX * 8 +                       // statx
         (size_t)C_WORDS * 4 +                               // ctl
         (size_t)2 * PTRACE_BLOCKS * 16 * 8;                 // phase timestamps
}

void persist_bind_scratch(PersistArgs& a, void* base) {
  char* p = (char*)base;
  a.hx = (float*)p;
  p += (size_t)NX * SMAX * PD * 4;
  a.qkvx = (uint16_t*)p;
  p += (size_t)NX * 3 * (PNH / NX) * SMAX * PHD * 2;
  a.ox = (uint16_t*)p;
  p += (size_t)NX * SMAX * AX * 2;
  a.ux = (uint16_t*)p;
  p += (size_t)NX * SMAX * FX * 2;
  a.part = (float*)p;
  p += (size_t)2 * NX * SMAX * PD * 4;
  a.statx = (float2*)p;
  p += (size_t)NX * NWG * SMAX * 8;
  a.ctl = (unsigned*)p;
  p += (size_t)C_WORDS * 4;
  a.trace = (unsigned long long*)p;
}

unsigned* persist_error_word(const PersistArgs& a) { return a.ctl + C_ERR; }

hipError_t persist_init() {
  return hipFuncSetAttribute((const void*)dit_b1_persist_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             159 * 1024);  // the rest of the 160 KB is the kernel's static LDS
}

hipError_t launch_dit_b1_persist(const PersistArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(persist_reset_kernel, dim3(1), dim3(256), 0, s, a.ctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dit_b1_persist_kernel, dim3(PG), dim3(NT), persist_lds_bytes(a.S, a.L), s, a);
  return hipGetLastError();
}

}  // namespace gr00t

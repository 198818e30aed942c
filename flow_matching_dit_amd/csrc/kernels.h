// Launch interface of the gfx950 kernels of the GR00T action head.
// Every launcher enqueues on the given stream and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr00t {

enum DType { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };
enum Act { ACT_NONE = 0, ACT_RELU = 1, ACT_SILU = 2, ACT_GELU = 3 };
enum EpiKind {
  EPI_STORE = 0,      // out[row, n] = act(v)            (fp32 or bf16 out)
  EPI_RESID_ADD = 1,  // out[row, n] += act(v)           (fp32 residual stream)
  EPI_HEADS = 2,      // scatter to head-major [b][head][pos][hd] buffers (act dtype)
  EPI_EULER = 3,      // out[row, n] += dt * act(v)      (fp32 Euler state)
  EPI_PARTIAL = 4     // out[split][row, n] = v          (fp32 split-K partial sums, bias in split 0)
};

// C[g, r, n] = sum_k A[g, r, k] * W[id_g][n, k]   (then * wscale[id_g][n] + bias[id_g][n])
// A row (g, r) lives at A + (g * a_gstride + a_row_off + r) * lda.
// W is packed [N][K] (K contiguous) per category; category = ids[g] (0 if ids == NULL).
struct GemmArgs {
  const void* A;
  long lda;
  long a_gstride;
  int a_row_off;
  const void* W;
  long w_cstride;
  const float* wscale;  // per-column fp32 scale of e4m3 weights, NULL otherwise
  long s_cstride;
  const float* bias;    // NULL = no bias
  long b_cstride;
  const int* ids;       // per-group category, NULL = category 0
  int rows;             // rows per group
  int N;
  int K;
  int groups;
  int k_per_split;      // set by the launcher
  const int* rows_dev;  // optional device row count (dense GEMMs): rows = min(rows, *rows_dev)
  // Optional LayerNorm of the A rows, folded into the skinny bf16 kernel (gemm_ln_fits): A is
  // then the fp32 residual stream [rows][K] (row stride lda); each row is normalised over its K
  // values (eps 1e-5), multiplied by (1 + scale) and shifted when ln_ada = [scale K | shift K]
  // is given, and rounded to bf16 as the GEMM stages it. One split only.
  int ln;
  const float* ln_ada;
  const float* ascale;  // W8A8 (launch_gemm_a8): per-row fp32 scales of the e4m3 A rows, NULL otherwise
  // Category buckets (bf16 MFMA GEMMs over many samples): group g of the launch is chunk g of
  // a counting sort of the samples by category (launch_bucket_ids): chunks[g] = (category,
  // first index into perm, samples, 0), no samples = nothing to do. Its rows are the `rows`
  // rows of each of those samples (sample s: A rows s * a_gstride + a_row_off + 0 .., output
  // group s), so the category's weights are read once per chunk instead of once per sample.
  // map_bytes: bytes of A the samples' rows span. NULL: group g is one sample.
  const int4* chunks;
  const int* perm;
  int chunk_cap;        // samples per chunk at most (chunk_cap * rows <= the tile's rows)
  long map_bytes;
};

struct Epi {
  int kind;
  int act;
  void* out;
  int out_f32;          // EPI_STORE: 1 = fp32 out, 0 = bf16 out
  long out_ld;          // row stride of out (elements)
  long out_gstride;     // rows between groups
  int out_row_off;
  const float* add_tab; // optional row added before the activation: row cat (or g, add_by_group)
  long add_cstride;
  int add_by_group;     // 1: add_tab row = group index g instead of the group's category
  // EPI_HEADS: column n -> section sec = n / width, which = sec % nwhich,
  // layer = sec / nwhich, head = (n % width) / hd, d = n % hd; row r -> (b, pos) with
  // pos_per_b positions per sample; element goes to heads[which] + layer * layer_stride[which] +
  //   ((b * nh + head) * pstride[which] + pos) * hd + d        (row-major positions), or
  //   (b * nh + head) * pstride[which] * hd + (pos / 32) * hd * 32 + d * 32 + pos % 32
  //                                                 (transposed[which]: [pos / 32][hd][pos % 32];
  //                                                  pstride a multiple of 32).
  void* heads[3];
  int nwhich;
  int width;
  int nh;
  int hd;
  int pos_per_b;
  int pstride[3];
  int transposed[3];
  long layer_stride[3];
  const int* row_map;   // EPI_HEADS: optional map of the GEMM row to the (b * pos_per_b + pos) row
  float dt;             // EPI_EULER
  int splits;           // EPI_PARTIAL: number of K splits (grid z)
  long split_stride;    // EPI_PARTIAL: elements between consecutive splits' outputs
};

hipError_t launch_gemm_valu(const GemmArgs& a, const Epi& e, DType at, DType wt, hipStream_t s);
hipError_t launch_gemm_mfma(const GemmArgs& a, const Epi& e, DType wt, hipStream_t s);
// W8A8: e4m3 A rows (a.A, row stride a.lda bytes, row scales a.ascale) times e4m3 weights (a.W,
// column scales a.wscale) on the gfx950 16x16x128 fp8 MFMA, fp32 accumulation, the epilogue e.
// Dense (one group), K % 16 == 0, splits as launch_gemm_mfma.
hipError_t launch_gemm_a8(const GemmArgs& a, const Epi& e, hipStream_t s);
// Whether a GEMM of `rows` rows and depth K with weights wt can take its A rows through the
// folded LayerNorm (GemmArgs::ln): at most 32 rows, bf16 weights, 1024 <= K <= 2048, K a
// multiple of 256, and the staged rows within the kernel's LDS budget.
bool gemm_ln_fits(int rows, int K, DType wt);
// K splits the MFMA GEMM would use for a split-K launch of this shape (1 = none); bf16w:
// bf16 weights (few rows may then take the staged-rows skinny kernel).
int gemm_mfma_splits(int rows, int N, int K, int groups, bool bf16w);

// LayerNorm over rows of width D (eps 1e-5, population variance):
//   y = (x - mean) / sqrt(var + eps) [* gamma + beta] [* (1 + scale) + shift]
// with ada = [scale | shift] (2D floats) or NULL. x rows at x + r * ldx.
hipError_t launch_layernorm(const void* x, DType xt, long ldx, void* y, DType yt, long ldy, int rows,
                            int D, const float* gamma, const float* beta, const float* ada,
                            hipStream_t s, const int* row_idx = nullptr, const int* row_count = nullptr);
// With row_idx/row_count: output row r (< *row_count) is the normalised input row row_idx[r].

// idx[0 .. *count) = the rows r < n with code[r] != 0, in increasing order (one workgroup).
hipError_t launch_compact_rows(const uint8_t* code, int n, int* idx, int* count, hipStream_t s);

// Residual add of split-K partial sums, then adaLN / LayerNorm:
//   h[r] += sum_s partials[s][r]  (fixed order, written back), y = LN(h[r]) [* (1 + scale) + shift]
// partials may be NULL (nsplit = 0): then it is launch_layernorm on fp32 h.
// ada_rows > 0: row r takes its modulation from ada + (r / ada_rows) * ada_stride (one
// [scale | shift] per sample of ada_rows rows); 0: every row uses ada.
// yt = DT_FP8 (W8A8): y receives the e4m3 codes [rows][D] of the bf16-rounded output and
// qscale[rows] their row scales, as launch_quant_rows would make them from a bf16 y.
hipError_t launch_resid_layernorm(float* h, const float* partials, int nsplit, long split_stride, void* y,
                                  DType yt, int rows, int D, const float* ada, hipStream_t s, int ada_rows = 0,
                                  long ada_stride = 0, float* qscale = nullptr);

// Multi-head attention per (sample, head): softmax(q k^T / sqrt(hd)) v.
// q [B][nh][S][hd]; k [B][nh][Lp][hd] (keys row-major, Lp = Lk rounded up to 32);
// vt [B][nh][Lp/32][hd][32] (values transposed per 32-key tile); o [B*S][nh*hd]; all in act dtype. Key rows
// and value columns in [Lk, Lp) must hold finite values (they get weight 0).
// mask: NULL = every key admitted; else key j of sample b is admitted iff
// (mask[b * Lk + j] & mask_bit) != 0. A query with no admitted key outputs 0.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  const uint8_t* mask;
  int mask_bit;
  int B, S, Lk, Lp, nh, hd;
};
hipError_t launch_attention(const AttnArgs& a, DType t, hipStream_t s);

// Small kernels.
// code[b*L + j] = bit0: admitted on text-attending blocks, bit1: on image-attending
// blocks. Without an image mask both bits equal the valid bit.
hipError_t launch_mask_codes(const uint8_t* vl_mask, const uint8_t* image_mask, uint8_t* code, int n,
                             hipStream_t s);
// ids_out[b] = ids_in[b] if in [0, C) else 0; bad[b] = out of range; *bad_count (when given) is
// increased by the number of out-of-range ids (a monotonic count across calls).
// Counting sort of the B sanitised ids (in [0, C)) by category, stable: perm lists the samples
// of category 0 in sample order, then category 1, ...; chunks[j] (j < maxch = ceil(B / cap) +
// min(B, C)) splits each category's run into runs of at most cap samples, (category, first
// index into perm, samples, 0), the unused entries (0, 0, 0, 0). One workgroup.
hipError_t launch_bucket_ids(const int* ids, int B, int C, int cap, int* perm, int4* chunks, hipStream_t s);
inline int bucket_max_chunks(int B, int C, int cap) { return (B + cap - 1) / cap + (B < C ? B : C); }
hipError_t launch_sanitize_ids(const int* ids_in, int* ids_out, uint8_t* bad, int B, int C,
                               hipStream_t s, unsigned* bad_count = nullptr);
// dst rows (b * dst_stride_rows + dst_row_off) <- src rows b (fp32, width D).
hipError_t launch_copy_rows(const float* src, long src_ld, float* dst, long dst_ld, long dst_gstride,
                            int dst_row_off, int B, int D, hipStream_t s);
// x = noise (n floats), or N(0,1) from Philox4x32-10 + Box-Muller when noise == NULL.
hipError_t launch_init_noise(const float* noise, float* x, long n, uint64_t seed, uint64_t counter,
                             hipStream_t s);
// out[b, i] = bad[b] ? NaN : x[b, i] * (mask ? mask[b, i] : 1), per = H*A.
hipError_t launch_output(const float* x, const uint8_t* mask, const uint8_t* bad, float* out, int B,
                         int per, hipStream_t s);
// tab[k][i] = sinusoid(tau[k]) of width dim: [sin(tau w_i) | cos(tau w_i)], w_i = 10000^(-i/half).
hipError_t launch_sinusoid(const int* tau_host_k, int K, int dim, float* tab, hipStream_t s);
// tab[b] = sinusoid (as launch_sinusoid) of the bucket floor(t[b] * buckets), decided in fp32, b < n.
hipError_t launch_sinusoid_t(const float* t, int n, int buckets, int dim, float* tab, hipStream_t s);
// x[b, i] = (1 - t[b]) * noise[b, i] + t[b] * actions[b, i], per values per sample.
hipError_t launch_flow_interp(const float* actions, const float* noise, const float* t, float* x, int B, int per,
                              hipStream_t s);
// loss[0] = sum(mask * (v_pred - (actions - noise))^2) / (sum(mask) + 1e-6) over B * per values (mask NULL:
// ones), summed in double in a fixed order (one workgroup); NaN if bad[b] != 0 for some sample.
hipError_t launch_masked_mse(const float* v_pred, const float* actions, const float* noise, const uint8_t* mask,
                             const uint8_t* bad, int B, int per, float* loss, hipStream_t s);
// W8A8: bf16 rows x [rows][K] (row stride ldx) -> e4m3 codes q (row stride ldq, bytes) and fp32
// row scales: scale[r] = amax_r / 448 (1 for an all-zero row), q = e4m3(x / scale) (nearest, ties
// to even, saturating). Rows >= *rows_dev are skipped when rows_dev is given. K, ldx, ldq % 8 == 0.
hipError_t launch_quant_rows(const void* x, long ldx, int rows, int K, uint8_t* q, long ldq, float* scale,
                             hipStream_t s, const int* rows_dev = nullptr);
// y = SiLU(x), n floats.
hipError_t launch_silu(const float* x, float* y, long n, hipStream_t s);
// fp32 -> act dtype copy of n elements.
hipError_t launch_convert(const float* x, void* y, DType yt, long n, hipStream_t s);

// ------------------------------------------------------------------ persistent B = 1 blocks
// Weights of one DiT block as the persistent kernel reads them (packed [out][in] bf16).
struct PBlock {
  const uint16_t* wq;  // [nq * D][D]: q (cross blocks, nq = 1) or q; k; v (self blocks, nq = 3)
  const float* bq;     // [nq * D]
  const uint16_t* wo;  // [D][D]
  const float* bo;     // [D]
  const uint16_t* w1;  // [F][D]
  const float* b1;     // [F]
  const uint16_t* w2;  // [D][F]
  const float* b2;     // [D]
  int nq;
};

// One Euler step's DiT blocks for one sample in one launch (persist.hip): D = 1536 (32 heads
// of 48), F = 6144, S <= 32 rows, on a device of 256 CUs in 8 XCDs.
struct PersistArgs {
  const PBlock* blocks;  // [nl] (device)
  int nl;
  int S;                 // rows: the state token and H action tokens
  float* h;              // [S][D] fp32 residual stream: the blocks' input, replaced by their output
  const float* ada;      // [nl][2D] adaLN [scale | shift] of every block at this step
  const uint16_t* kc;    // key cache of the cross blocks [cross block][head][Lp][hd] (B = 1)
  const uint16_t* vc;    // value cache [cross block][head][Lp / 32][hd][32]
  long kv_layer;         // elements between two cross blocks' caches
  const uint8_t* code;   // [L] key mask codes: bit 0 text blocks, bit 1 image blocks
  int L, Lp, text_every;
  // scratch (persist_scratch_bytes, bound by persist_bind_scratch)
  float* hx;
  uint16_t* qkvx;
  uint16_t* ox;
  uint16_t* ux;
  float* part;
  float2* statx;
  unsigned* ctl;
  unsigned long long* trace;  // phase timestamps (written by GR00T_PHASE_TRACE builds only)
  unsigned spin;              // polls before a wait gives up (0: 2^20)
};
// Words of the phase timestamp area (2 workgroups x 64 blocks x 16 boundaries).
constexpr int persist_trace_words() { return 2 * 64 * 16; }
// Whether the persistent kernel serves this shape (model widths, rows, VL length, CU count).
bool persist_b1_fits(int D, int F, int nh, int hd, int S, int L, int num_cus);
size_t persist_scratch_bytes();
void persist_bind_scratch(PersistArgs& a, void* base);
// device word counting the persistent kernel's timed-out waits (never cleared)
unsigned* persist_error_word(const PersistArgs& a);
// allows the kernel its dynamic LDS (once per process, before the first launch)
hipError_t persist_init();
// scratch.hip: the fixed device scratch area of the entry points that do not allocate
size_t static_scratch_bytes();
hipError_t static_scratch_address(int device, void** ptr);  // `device` must be current
// clears the control words, then launches the kernel (two launches on s)
hipError_t launch_dit_b1_persist(const PersistArgs& a, hipStream_t s);

}  // namespace gr00t

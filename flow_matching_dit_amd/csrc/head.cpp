// Host runtime of the GR00T action head behind the C ABI of gr00t_head.h.
//
// Owns: argument validation (no HIP call before a check passes), the weight
// registry and packer (fp32 masters -> bf16 round-to-nearest-even or per-column
// e4m3, transposed to the [out][in] layout the GEMM kernels read), the device
// arena, the workspace, the per-step tables, and the launch sequence of one
// get_action call:
//   prologue  : mask codes, id check, vision-language LayerNorm, the key/value
//               projection of every cross-attention block (once per call, reused by
//               all K steps), the state encoder, x0 = noise;
//   K steps   : action encoder -> state+action tokens -> 32 DiT blocks -> output
//               adaLN + projection -> decoder with the Euler update fused in;
//   epilogue  : action_pred = x * action_mask.
// The K-step part can be captured once per (B, L_pad) into a hipGraph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <thread>
#include <tuple>
#include <utility>
#include <vector>

#include "gr00t_head.h"
#include "kernels.h"

using namespace gr00t;

namespace {

thread_local std::string g_create_error;

// ------------------------------------------------------------------ host number formats

uint16_t host_f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

float host_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Nearest OCP E4M3 code of a (finite) float, ties to even, magnitudes >= 448 saturate.
uint8_t host_f32_to_e4m3(float v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0;
  const float a = std::fabs(v);
  if (!(a < 448.0f)) return sign | 0x7E;
  if (a < 0.015625f) {  // below 2^-6: subnormal quantum 2^-9
    const int m = (int)std::nearbyint(a * 512.0f);  // 0..8; 8 is the smallest normal
    return sign | (uint8_t)m;
  }
  int e;
  std::frexp(a, &e);  // a in [2^(e-1), 2^e)
  int E = e - 1;      // -6 .. 8
  int mq = (int)std::nearbyint(std::ldexp(a, 3 - E));  // 8 .. 16
  if (mq == 16) {
    mq = 8;
    E += 1;
  }
  return sign | (uint8_t)(((E + 7) << 3) | (mq - 8));
}

// ------------------------------------------------------------------ weight registry

enum Store { ST_F32 = 0, ST_BF16 = 1, ST_FP8 = 2 };

struct Piece {           // one packed destination of a loaded tensor
  size_t off = 0;        // byte offset of the packed data in the arena
  size_t scale_off = 0;  // byte offset of the per-column scales (ST_FP8)
  int in_lo = 0, in_n = 0;  // slice of the `in` axis taken (matrices)
};

struct Spec {
  std::vector<int64_t> shape;
  bool matrix = false;   // [.., in, out] linear weight, packed [C][out][in]
  Store store = ST_F32;  // storage of the packed data (vectors are always fp32)
  std::vector<Piece> pieces;
  bool loaded = false;
  std::vector<uint8_t> staged;  // packed bytes, per piece concatenated (data then scales)
};

struct LayerOff {
  size_t wq = 0, bq = 0, sq = 0;  // self: wq region = [Wq;Wk;Wv] (3D x D), biases/scales 3D
  size_t wo = 0, bo = 0, so = 0;
  size_t w1 = 0, b1 = 0, s1 = 0;
  size_t w2 = 0, b2 = 0, s2 = 0;
};

struct Layout {
  size_t vlln_g, vlln_b;
  size_t t_w1, t_b1, t_w2, t_b2;
  size_t se_w1, se_b1, se_w2, se_b2;
  size_t ae_w1, ae_b1, ae_w2a, ae_w2t, ae_b2, ae_w3, ae_b3;
  size_t ada_w, ada_b;
  std::vector<LayerOff> L;
  size_t kv_w, kv_b, kv_s;
  size_t p_w, p_b, p_s;
  size_t d_w1, d_b1, d_w2, d_b2;
  size_t total;
};

struct Ws {  // workspace pointers
  float* h;
  void *n, *q, *k, *v, *o, *u, *y, *e1, *e2, *se1, *vln, *kc, *vc;
  float *x, *s, *vout, *part;
  uint8_t *code, *bad;
  unsigned* bad_count;  // monotonic count of invalid ids met on the device (never cleared)
  int *ids, *iota, *vrow, *vcount;
  float *sin_t, *t1, *temb, *stemb, *ada, *tauemb, *c2tab;
  uint8_t* q8;  // W8A8: e4m3 input rows of the current GEMM
  float* qs;    // W8A8: their row scales
  int* perm;    // category buckets: the samples sorted by category
  int4* chunks; //   and the runs of at most kBucketCap samples of one category
};

// Batches of at least kBucketMinBatch samples run the per-embodiment bf16 GEMMs over category
// buckets of at most kBucketCap samples (one 128-row tile of 16-row samples): each category's
// weights are read once per bucket instead of once per sample.
constexpr int kBucketCap = 8, kBucketMinBatch = 128;

}  // namespace

// Shape and buffers of a get_action call: a captured whole call replays with exactly these.
struct CallKey {
  int B = 0, L = 0;
  std::array<const void*, 9> p{};
  bool operator<(const CallKey& o) const { return std::tie(B, L, p) < std::tie(o.B, o.L, o.p); }
  bool operator==(const CallKey& o) const { return B == o.B && L == o.L && p == o.p; }
};
constexpr size_t kMaxCallGraphs = 8;

struct gr00t_head {
  gr00t_config cfg{};
  int device = 0;
  std::string err;
  bool finalized = false;
  DType act = DT_BF16;
  std::map<std::string, Spec> specs;
  std::vector<std::string> order;
  Layout lay{};
  char* arena = nullptr;
  char* wsbase = nullptr;
  size_t ws_bytes = 0;
  Ws w{};
  hipStream_t cap_stream = nullptr;
  std::map<std::pair<int, int>, hipGraphExec_t> graphs;
  // whole-call graphs (prologue, K steps, output) keyed by the call's shape and buffers; the
  // buffers of the previous call (a call whose buffers repeat is captured)
  std::map<CallKey, hipGraphExec_t> call_graphs;
  std::vector<CallKey> call_order;  // capture order, for eviction
  CallKey last_call{};
  uint64_t calls = 0;
  // Deferred report of invalid ids (non-strict mode). Every call copies the device count of
  // invalid ids met so far and its per-sample flags into the next of kReportSlots pinned slots
  // and records an event. The count only grows, so any completed copy taken after a bad call
  // shows it, however many calls were enqueued in between; a count above bad_reported is
  // reported once by the next call that finds such a completed copy.
  static constexpr int kReportSlots = 4;
  struct ReportSlot {
    uint8_t* host = nullptr;  // [4 bytes invalid-id count][4 bytes block-kernel timeouts][max_batch flags]
    hipEvent_t ev = nullptr;
    bool recorded = false;
    int B = 0;
  } rep[kReportSlots];
  int rep_next = 0;
  uint32_t bad_reported = 0;
  // persistent kernel for the DiT blocks at B = 1 (persist.hip): usable for this model and
  // device, its scratch, the per-block weight table, and the timeouts already reported
  bool persist_ok = false;
  void* persist_base = nullptr;
  PBlock* persist_blocks = nullptr;
  uint32_t persist_err_reported = 0;
  // polls before one of its waits gives up (0: the kernel's default); GR00T_PERSIST_SPIN at
  // create, for tests of the fallback
  unsigned persist_spin = 0;
  // (B, L_pad) of the VL key/value caches and key masks in the workspace: those of the last
  // call that ran the full prologue (0, 0: none yet)
  int kv_B = 0, kv_L = 0;
  // per-sample timestep tables of the training forward (allocated on its first call)
  struct {
    float *sin_t = nullptr, *tauemb = nullptr, *t1 = nullptr, *temb = nullptr, *stemb = nullptr, *ada = nullptr,
          *c2 = nullptr;
  } tr;
  void* tr_base = nullptr;
  // device address of the library's fixed scratch area on this handle's device (scratch.hip),
  // looked up at finalize: the per-sample tables of gr00t_train_forward_noalloc
  void* static_scratch = nullptr;
  std::vector<int> tau;
  // launch timing (gr00t_profile_*)
  bool prof_on = false;
  int prof_mode = 0;  // 1: every launch, eager; 2: graph kept, launches outside it timed
  std::vector<hipEvent_t> prof_pool;
  std::vector<std::pair<int, int>> prof_recs;  // (class, index of the start event)
  size_t prof_next = 0;
  std::vector<int64_t> prof_n;
  std::vector<double> prof_ms;
};

namespace {

int fail(gr00t_head* h, int code, const std::string& msg) {
  if (h) h->err = msg;
  return code;
}

size_t act_bytes(const gr00t_head* h) { return h->act == DT_F32 ? 4 : 2; }

int round32(int x) { return (x + 31) / 32 * 32; }


std::string shape_str(const std::vector<int64_t>& s) {
  std::string r = "[";
  for (size_t i = 0; i < s.size(); ++i) r += (i ? "," : "") + std::to_string(s[i]);
  return r + "]";
}

int check_config(const gr00t_config* c, std::string& why) {
  if (!c) { why = "config is NULL"; return GR00T_E_INVALID_ARG; }
  auto bad = [&](const char* m) { why = m; return GR00T_E_INVALID_ARG; };
  if (c->num_layers < 1) return bad("num_layers must be >= 1");
  if (c->num_heads < 1 || c->head_dim < 16 || c->head_dim > 64 || c->head_dim % 16)
    return bad("head_dim must be a multiple of 16 in [16, 64]");
  if (c->hidden != c->num_heads * c->head_dim) return bad("hidden must equal num_heads * head_dim");
  if (c->hidden > 2048 || c->hidden % 16) return bad("hidden must be a multiple of 16, at most 2048");
  if (c->vl_dim < 16 || c->vl_dim > 2048 || c->vl_dim % 16) return bad("vl_dim must be a multiple of 16 in [16, 2048]");
  if (c->ff_dim < 16 || c->ff_dim % 16) return bad("ff_dim must be a positive multiple of 16");
  if (c->state_dim < 1) return bad("state_dim must be >= 1");
  if (c->action_dim < 1) return bad("action_dim must be >= 1");
  if (c->action_horizon < 1 || c->action_horizon + 1 > 65) return bad("action_horizon must be in [1, 64]");
  if (c->num_categories < 1) return bad("num_categories must be >= 1");
  if (c->num_steps < 1 || c->num_steps > 64) return bad("num_steps must be in [1, 64]");
  if (c->num_timestep_buckets < 1) return bad("num_timestep_buckets must be >= 1");
  if (c->attend_text_every_n_blocks < 1) return bad("attend_text_every_n_blocks must be >= 1");
  if (c->time_freq_dim < 2 || c->time_freq_dim % 2) return bad("time_freq_dim must be even and >= 2");
  if (c->max_batch < 1 || c->max_vl_len < 1) return bad("max_batch and max_vl_len must be >= 1");
  if (!(c->weight_dtype == GR00T_F32 || c->weight_dtype == GR00T_BF16 || c->weight_dtype == GR00T_FP8_E4M3))
    return bad("weight_dtype must be F32, BF16 or FP8_E4M3");
  if (!(c->act_dtype == GR00T_F32 || c->act_dtype == GR00T_BF16)) return bad("act_dtype must be F32 or BF16");
  if ((c->weight_dtype == GR00T_F32) != (c->act_dtype == GR00T_F32))
    return bad("F32 weights go with F32 activations, BF16/FP8 weights with BF16 activations");
  if (c->flags & ~(GR00T_FLAG_STRICT | GR00T_FLAG_USE_GRAPH | GR00T_FLAG_W8A8 | GR00T_FLAG_PERSIST |
                   GR00T_FLAG_NO_BUCKETS))
    return bad("unknown flag bits");
  if ((c->flags & GR00T_FLAG_W8A8) && c->weight_dtype != GR00T_FP8_E4M3)
    return bad("GR00T_FLAG_W8A8 needs FP8_E4M3 weights");
  // The kernels address each GEMM operand, cache layer and workspace buffer through a 32-bit
  // buffer descriptor with 32-bit offsets: every such operand must stay below 2^31 - 16 bytes.
  {
    const double Bm = c->max_batch, Lm = c->max_vl_len, Lmp = (c->max_vl_len + 31) / 32 * 32.0;
    const double D = c->hidden, F = c->ff_dim, E = c->vl_dim, S = c->action_horizon + 1.0;
    const double C = c->num_categories, Nl = c->num_layers, Nc = (c->num_layers + 1) / 2;
    const double ab = c->act_dtype == GR00T_F32 ? 4.0 : 2.0, wb = c->weight_dtype == GR00T_F32 ? 4.0 : 2.0;
    const double limit = 2147483632.0;  // 0x7FFFFFF0
    const struct { const char* what; double bytes; } ops[] = {
        {"the VL features and K/V projection input (max_batch * max_vl_len * vl_dim)", Bm * Lm * E * ab},
        {"one cross block's key or value cache (max_batch * max_vl_len * hidden)", Bm * Lmp * D * ab},
        {"the MLP activations (max_batch * (action_horizon + 1) * ff_dim)", Bm * S * F * ab},
        {"the split-K partial sums (8 * max_batch * (action_horizon + 1) * hidden)", 8.0 * Bm * S * D * 4.0},
        {"the K/V projection weights (cross blocks * 2 * hidden * vl_dim)", Nc * 2.0 * D * E * wb},
        {"one MLP weight matrix (ff_dim * hidden)", F * D * wb},
        {"the adaLN weights ((num_layers + 1) * 2 * hidden * hidden)", (Nl + 1.0) * 2.0 * D * D * wb},
        {"one per-embodiment weight table (num_categories * hidden * hidden)", C * D * D * wb},
    };
    for (const auto& o : ops)
      if (o.bytes > limit) {
        why = std::string("capacity too large: ") + o.what + " would take " + std::to_string((long long)o.bytes) +
              " bytes, above the 2^31 - 16 bytes one buffer descriptor addresses";
        return GR00T_E_INVALID_ARG;
      }
  }
  return GR00T_OK;
}

bool is_fp8_name(const std::string& n) {
  if (n == "out.proj.w") return true;
  if (n.rfind("blocks.", 0) != 0) return false;
  static const char* suf[] = {"attn.wq", "attn.wk", "attn.wv", "attn.wo", "ff.w1", "ff.w2"};
  for (const char* s : suf) {
    const size_t ls = std::strlen(s);
    if (n.size() >= ls && n.compare(n.size() - ls, ls, s) == 0) return true;
  }
  return false;
}

// Build the canonical weight list and the arena layout for the config.
void build_specs(gr00t_head* h) {
  const gr00t_config& c = h->cfg;
  const int64_t D = c.hidden, F = c.ff_dim, C = c.num_categories, E = c.vl_dim, Nl = c.num_layers;
  const int Nc = (int)((Nl + 1) / 2);
  const Store mat = c.weight_dtype == GR00T_F32 ? ST_F32 : ST_BF16;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  auto elt = [&](Store s) -> size_t { return s == ST_F32 ? 4 : (s == ST_BF16 ? 2 : 1); };
  auto add = [&](const std::string& name, std::vector<int64_t> shape, bool matrix) -> Spec& {
    Spec& s = h->specs[name];
    s.shape = std::move(shape);
    s.matrix = matrix;
    s.store = matrix ? ((c.weight_dtype == GR00T_FP8_E4M3 && is_fp8_name(name)) ? ST_FP8 : mat) : ST_F32;
    h->order.push_back(name);
    return s;
  };
  auto vec = [&](const std::string& name, std::vector<int64_t> shape, size_t at) {
    Spec& s = add(name, shape, false);
    Piece p;
    p.off = at;
    s.pieces.push_back(p);
  };
  auto matp = [&](const std::string& name, std::vector<int64_t> shape, size_t at, size_t sat, int in_lo, int in_n) {
    Spec& s = h->specs[name];
    if (s.shape.empty()) add(name, shape, true);
    Piece p;
    p.off = at;
    p.scale_off = sat;
    p.in_lo = in_lo;
    p.in_n = in_n;
    h->specs[name].pieces.push_back(p);
  };
  Layout& L = h->lay;
  L.L.resize(Nl);
  const size_t me = elt(mat);
  const auto mstore = [&](const std::string& n) { return (c.weight_dtype == GR00T_FP8_E4M3 && is_fp8_name(n)) ? ST_FP8 : mat; };

  L.vlln_g = take(E * 4); vec("vlln.gamma", {E}, L.vlln_g);
  L.vlln_b = take(E * 4); vec("vlln.beta", {E}, L.vlln_b);
  L.t_w1 = take((size_t)c.time_freq_dim * D * me); matp("time.w1", {c.time_freq_dim, D}, L.t_w1, 0, 0, c.time_freq_dim);
  L.t_b1 = take(D * 4); vec("time.b1", {D}, L.t_b1);
  L.t_w2 = take(D * D * me); matp("time.w2", {D, D}, L.t_w2, 0, 0, (int)D);
  L.t_b2 = take(D * 4); vec("time.b2", {D}, L.t_b2);
  L.se_w1 = take(C * c.state_dim * D * me); matp("state_enc.w1", {C, c.state_dim, D}, L.se_w1, 0, 0, c.state_dim);
  L.se_b1 = take(C * D * 4); vec("state_enc.b1", {C, D}, L.se_b1);
  L.se_w2 = take(C * D * D * me); matp("state_enc.w2", {C, D, D}, L.se_w2, 0, 0, (int)D);
  L.se_b2 = take(C * D * 4); vec("state_enc.b2", {C, D}, L.se_b2);
  L.ae_w1 = take(C * c.action_dim * D * me); matp("action_enc.w1", {C, c.action_dim, D}, L.ae_w1, 0, 0, c.action_dim);
  L.ae_b1 = take(C * D * 4); vec("action_enc.b1", {C, D}, L.ae_b1);
  L.ae_w2a = take(C * D * D * me);
  L.ae_w2t = take(C * D * D * me);
  matp("action_enc.w2", {C, 2 * D, D}, L.ae_w2a, 0, 0, (int)D);
  matp("action_enc.w2", {C, 2 * D, D}, L.ae_w2t, 0, (int)D, (int)D);
  L.ae_b2 = take(C * D * 4); vec("action_enc.b2", {C, D}, L.ae_b2);
  L.ae_w3 = take(C * D * D * me); matp("action_enc.w3", {C, D, D}, L.ae_w3, 0, 0, (int)D);
  L.ae_b3 = take(C * D * 4); vec("action_enc.b3", {C, D}, L.ae_b3);
  // adaLN linears of all blocks and of the output norm, concatenated along N.
  L.ada_w = take((size_t)(Nl + 1) * 2 * D * D * me);
  L.ada_b = take((size_t)(Nl + 1) * 2 * D * 4);
  // cross key/value projections of all cross blocks, concatenated along N.
  const Store kvs = mstore("blocks.0.attn.wk");
  L.kv_w = take((size_t)Nc * 2 * D * E * elt(kvs));
  L.kv_b = take((size_t)Nc * 2 * D * 4);
  L.kv_s = take((size_t)Nc * 2 * D * 4);
  for (int l = 0; l < Nl; ++l) {
    const std::string p = "blocks." + std::to_string(l) + ".";
    LayerOff& lo = L.L[l];
    const size_t esz = elt(mstore(p + "attn.wq"));
    matp(p + "ada.w", {D, 2 * D}, L.ada_w + (size_t)l * 2 * D * D * me, 0, 0, (int)D);
    vec(p + "ada.b", {2 * D}, L.ada_b + (size_t)l * 2 * D * 4);
    const bool self = (l % 2) == 1;
    const int nq = self ? 3 : 1;
    lo.wq = take((size_t)nq * D * D * esz);
    lo.bq = take((size_t)nq * D * 4);
    lo.sq = take((size_t)nq * D * 4);
    matp(p + "attn.wq", {D, D}, lo.wq, lo.sq, 0, (int)D);
    vec(p + "attn.bq", {D}, lo.bq);
    if (self) {
      matp(p + "attn.wk", {D, D}, lo.wq + (size_t)D * D * esz, lo.sq + D * 4, 0, (int)D);
      vec(p + "attn.bk", {D}, lo.bq + D * 4);
      matp(p + "attn.wv", {D, D}, lo.wq + (size_t)2 * D * D * esz, lo.sq + 2 * D * 4, 0, (int)D);
      vec(p + "attn.bv", {D}, lo.bq + 2 * D * 4);
    } else {
      const int ci = l / 2;
      const size_t kesz = elt(kvs);
      matp(p + "attn.wk", {E, D}, L.kv_w + (size_t)(2 * ci) * D * E * kesz, L.kv_s + (size_t)(2 * ci) * D * 4, 0,
           (int)E);
      vec(p + "attn.bk", {D}, L.kv_b + (size_t)(2 * ci) * D * 4);
      matp(p + "attn.wv", {E, D}, L.kv_w + (size_t)(2 * ci + 1) * D * E * kesz,
           L.kv_s + (size_t)(2 * ci + 1) * D * 4, 0, (int)E);
      vec(p + "attn.bv", {D}, L.kv_b + (size_t)(2 * ci + 1) * D * 4);
    }
    lo.wo = take((size_t)D * D * esz); lo.bo = take(D * 4); lo.so = take(D * 4);
    matp(p + "attn.wo", {D, D}, lo.wo, lo.so, 0, (int)D);
    vec(p + "attn.bo", {D}, lo.bo);
    lo.w1 = take((size_t)F * D * esz); lo.b1 = take(F * 4); lo.s1 = take(F * 4);
    matp(p + "ff.w1", {D, F}, lo.w1, lo.s1, 0, (int)D);
    vec(p + "ff.b1", {F}, lo.b1);
    lo.w2 = take((size_t)D * F * esz); lo.b2 = take(D * 4); lo.s2 = take(D * 4);
    matp(p + "ff.w2", {F, D}, lo.w2, lo.s2, 0, (int)F);
    vec(p + "ff.b2", {D}, lo.b2);
  }
  matp("out.ada.w", {D, 2 * D}, L.ada_w + (size_t)Nl * 2 * D * D * me, 0, 0, (int)D);
  vec("out.ada.b", {2 * D}, L.ada_b + (size_t)Nl * 2 * D * 4);
  const size_t pe = elt(mstore("out.proj.w"));
  L.p_w = take(D * D * pe); L.p_b = take(D * 4); L.p_s = take(D * 4);
  matp("out.proj.w", {D, D}, L.p_w, L.p_s, 0, (int)D);
  vec("out.proj.b", {D}, L.p_b);
  L.d_w1 = take(C * D * D * me); matp("action_dec.w1", {C, D, D}, L.d_w1, 0, 0, (int)D);
  L.d_b1 = take(C * D * 4); vec("action_dec.b1", {C, D}, L.d_b1);
  L.d_w2 = take(C * D * c.action_dim * me); matp("action_dec.w2", {C, D, c.action_dim}, L.d_w2, 0, 0, (int)D);
  L.d_b2 = take(C * c.action_dim * 4); vec("action_dec.b2", {C, (int64_t)c.action_dim}, L.d_b2);
  L.total = off;
}

// Run f(i) for i in [0, n) on up to hardware_concurrency threads.
template <typename Fn>
void parallel_for(int64_t n, Fn f) {
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n < 2 || nt == 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&]() {
      for (int64_t i = next.fetch_add(1); i < n; i = next.fetch_add(1)) f(i);
    });
  for (auto& x : th) x.join();
}

// Pack a loaded tensor (fp32 values or raw bf16 bits) into its pieces. Matrices
// [C][IN][OUT] become [C][OUT][in_n] (the slice [in_lo, in_lo + in_n) of IN), in
// 64 x 64 blocks so both sides are read and written in cache lines.
void pack(gr00t_head* h, Spec& s, const void* data, gr00t_dtype dt) {
  const float* f32 = (const float*)data;
  const uint16_t* b16 = (const uint16_t*)data;
  auto val = [&](size_t i) -> float { return dt == GR00T_F32 ? f32[i] : host_bf16_to_f32(b16[i]); };
  size_t numel = 1;
  for (auto d : s.shape) numel *= (size_t)d;
  s.staged.clear();
  if (!s.matrix) {
    s.staged.resize(numel * 4);
    float* o = (float*)s.staged.data();
    const bool keep32 = h->cfg.weight_dtype == GR00T_F32;
    for (size_t i = 0; i < numel; ++i) o[i] = keep32 ? val(i) : host_bf16_to_f32(host_f32_to_bf16(val(i)));
    return;
  }
  const size_t nd = s.shape.size();
  const int64_t C = nd == 3 ? s.shape[0] : 1, IN = s.shape[nd - 2], OUT = s.shape[nd - 1];
  constexpr int64_t BLK = 64;
  for (const Piece& p : s.pieces) {
    const int64_t in_n = p.in_n;
    const size_t base = s.staged.size();
    const size_t esz = s.store == ST_F32 ? 4 : (s.store == ST_BF16 ? 2 : 1);
    const size_t nbytes = (size_t)C * OUT * in_n * esz + (s.store == ST_FP8 ? (size_t)C * OUT * 4 : 0);
    s.staged.resize(base + nbytes);
    uint8_t* dst = s.staged.data() + base;
    float* scales = (float*)(dst + (size_t)C * OUT * in_n);
    if (s.store == ST_FP8) {  // per-column scale = max |W[:, o]| / 448 (1 for an all-zero column)
      parallel_for(C, [&](int64_t cc) {
        std::vector<float> amax(OUT, 0.0f);
        for (int64_t i = 0; i < in_n; ++i) {
          const size_t row = (size_t)(cc * IN + p.in_lo + i) * OUT;
          for (int64_t oo = 0; oo < OUT; ++oo) amax[oo] = std::fmax(amax[oo], std::fabs(val(row + oo)));
        }
        for (int64_t oo = 0; oo < OUT; ++oo) scales[cc * OUT + oo] = amax[oo] > 0.0f ? amax[oo] / 448.0f : 1.0f;
      });
    }
    const int64_t nob = (OUT + BLK - 1) / BLK;
    parallel_for(C * nob, [&](int64_t task) {
      const int64_t cc = task / nob, o0 = (task % nob) * BLK, o1 = std::min(OUT, o0 + BLK);
      for (int64_t i0 = 0; i0 < in_n; i0 += BLK) {
        const int64_t i1 = std::min(in_n, i0 + BLK);
        for (int64_t oo = o0; oo < o1; ++oo) {
          const size_t drow = (size_t)(cc * OUT + oo) * in_n;
          for (int64_t i = i0; i < i1; ++i) {
            const size_t si = (size_t)(cc * IN + p.in_lo + i) * OUT + oo;
            if (s.store == ST_F32) {
              ((float*)dst)[drow + i] = val(si);
            } else if (s.store == ST_BF16) {
              ((uint16_t*)dst)[drow + i] = dt == GR00T_BF16 ? b16[si] : host_f32_to_bf16(val(si));
            } else {
              dst[drow + i] = host_f32_to_e4m3(val(si) / scales[cc * OUT + oo]);
            }
          }
        }
      }
    });
  }
}

#define HIPCHK(h, expr)                                                                                   \
  do {                                                                                                    \
    hipError_t e__ = (expr);                                                                              \
    if (e__ != hipSuccess)                                                                                \
      return fail((h), GR00T_E_HIP, std::string(#expr) + " failed: " + hipGetErrorString(e__));           \
  } while (0)

// ------------------------------------------------------------------ launch timing

enum KClass {
  K_VLLN = 0, K_KV_PROJ, K_STATE_ENC, K_ACTION_ENC, K_ADALN, K_QKV_PROJ, K_Q_PROJ, K_ATTN_SELF, K_ATTN_CROSS,
  K_O_PROJ, K_NORM3, K_FF_UP, K_FF_DOWN, K_OUT_PROJ, K_DECODER, K_SMALL, K_GRAPH, K_BLOCKS, K_CALL_GRAPH, K_NCLASS
};
const char* const kClassNames[K_NCLASS] = {"vlln", "kv_proj", "state_enc", "action_enc", "adaln", "qkv_proj",
                                           "q_proj", "attn_self", "attn_cross", "o_proj", "norm3", "ff_up",
                                           "ff_down", "out_proj", "decoder", "small", "steps_graph",
                                           "blocks_b1", "call_graph"};

// Returns the index of the start event recorded on s, or -1 when not profiling.
int prof_begin(gr00t_head* h, hipStream_t s) {
  if (!h->prof_on) return -1;
  while (h->prof_pool.size() < h->prof_next + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    h->prof_pool.push_back(e);
  }
  const int i = (int)h->prof_next;
  h->prof_next += 2;
  if (hipEventRecord(h->prof_pool[i], s) != hipSuccess) return -1;
  return i;
}

void prof_end(gr00t_head* h, hipStream_t s, int cls, int i) {
  if (i < 0) return;
  if (hipEventRecord(h->prof_pool[i + 1], s) == hipSuccess) h->prof_recs.emplace_back(cls, i);
}

int prof_collect(gr00t_head* h) {
  for (const auto& r : h->prof_recs) {
    HIPCHK(h, hipEventSynchronize(h->prof_pool[r.second + 1]));
    float ms = 0.0f;
    HIPCHK(h, hipEventElapsedTime(&ms, h->prof_pool[r.second], h->prof_pool[r.second + 1]));
    h->prof_n[r.first] += 1;
    h->prof_ms[r.first] += ms;
  }
  h->prof_recs.clear();
  h->prof_next = 0;
  return GR00T_OK;
}

#define LAUNCH(h, s, cls, expr)          \
  do {                                   \
    const int ev__ = prof_begin((h), (s)); \
    HIPCHK((h), (expr));                 \
    prof_end((h), (s), (cls), ev__);     \
  } while (0)

template <typename T>
T* at(gr00t_head* h, size_t off) {
  return (T*)(h->arena + off);
}

// ------------------------------------------------------------------ GEMM dispatch

GemmArgs ga(const void* A, long lda, int rows, int N, int K) {
  GemmArgs a{};
  a.A = A;
  a.lda = lda;
  a.rows = rows;
  a.N = N;
  a.K = K;
  a.groups = 1;
  return a;
}

Epi ep_store(void* out, bool f32, long ld, int act = ACT_NONE) {
  Epi e{};
  e.kind = EPI_STORE;
  e.act = act;
  e.out = out;
  e.out_f32 = f32 ? 1 : 0;
  e.out_ld = ld;
  return e;
}

// W8A8: quantise the bf16 input rows to e4m3 (one scale per row), then the fp8 x fp8 GEMM
hipError_t gemm_a8(gr00t_head* h, const GemmArgs& a_in, const Epi& e, hipStream_t s) {
  GemmArgs a = a_in;
  hipError_t r = launch_quant_rows(a.A, a.lda, a.rows, a.K, h->w.q8, a.K, h->w.qs, s, a.rows_dev);
  if (r != hipSuccess) return r;
  a.A = h->w.q8;
  a.lda = a.K;
  a.ascale = h->w.qs;
  return launch_gemm_a8(a, e, s);
}

bool use_a8(const gr00t_head* h, DType at, DType wt) {
  return (h->cfg.flags & GR00T_FLAG_W8A8) && at == DT_BF16 && wt == DT_FP8;
}

// W8A8 GEMM whose input rows a LayerNorm has already written as e4m3 codes and row scales
hipError_t gemm_q8(gr00t_head* h, const GemmArgs& a_in, const Epi& e, hipStream_t s) {
  GemmArgs a = a_in;
  a.A = h->w.q8;
  a.lda = a.K;
  a.ascale = h->w.qs;
  return launch_gemm_a8(a, e, s);
}

bool use_buckets(const gr00t_head* h, int B) {
  return !(h->cfg.flags & GR00T_FLAG_NO_BUCKETS) && B >= kBucketMinBatch && h->act == DT_BF16 &&
         h->cfg.weight_dtype != GR00T_F32;
}

hipError_t gemm(gr00t_head* h, const GemmArgs& a, const Epi& e, DType at, DType wt, hipStream_t s) {
  if (use_a8(h, at, wt)) return gemm_a8(h, a, e, s);
  if (at == DT_BF16 && (wt == DT_BF16 || wt == DT_FP8) && a.K % 16 == 0 && a.lda % 8 == 0 && a.N % 4 == 0) {
    // one group per sample with the sample's category (per-embodiment linear): over buckets
    if (wt == DT_BF16 && a.groups > 1 && a.ids == h->w.ids && use_buckets(h, a.groups) &&
        (e.kind == EPI_STORE || e.kind == EPI_EULER) && a.rows * kBucketCap <= 128) {
      GemmArgs b = a;
      b.chunks = h->w.chunks;
      b.perm = h->w.perm;
      b.chunk_cap = kBucketCap;
      b.groups = bucket_max_chunks(a.groups, h->cfg.num_categories, kBucketCap);
      b.ids = nullptr;
      b.map_bytes = ((long)(a.groups - 1) * a.a_gstride + a.a_row_off + a.rows) * a.lda * 2;
      return launch_gemm_mfma(b, e, wt, s);
    }
    return launch_gemm_mfma(a, e, wt, s);
  }
  return launch_gemm_valu(a, e, at, wt, s);
}

// h += A W^T + b for the residual stream h: direct residual add, or split-K into the
// partial buffer (then *pend = number of partials the next norm must add). direct: never split.
hipError_t resid_gemm(gr00t_head* h, const GemmArgs& a, DType at, DType wt, long pstride, int& pend, hipStream_t s,
                      bool direct = false) {
  Epi e = ep_store(h->w.h, true, a.N);
  const bool mfma = at == DT_BF16 && (wt == DT_BF16 || wt == DT_FP8) && a.K % 16 == 0 && a.lda % 8 == 0 &&
                    a.N % 4 == 0;
  const int splits = mfma && !direct ? gemm_mfma_splits(a.rows, a.N, a.K, a.groups, wt == DT_BF16) : 1;
  if (splits > 1) {
    e.kind = EPI_PARTIAL;
    e.out = h->w.part;
    e.splits = splits;
    e.split_stride = pstride;
    pend = splits;
    return use_a8(h, at, wt) ? gemm_a8(h, a, e, s) : launch_gemm_mfma(a, e, wt, s);
  }
  e.kind = EPI_RESID_ADD;
  pend = 0;
  return gemm(h, a, e, at, wt, s);
}

// ------------------------------------------------------------------ tables (finalize)

int build_tables(gr00t_head* h, hipStream_t s) {
  const gr00t_config& c = h->cfg;
  const int D = c.hidden, K = c.num_steps, Nl = c.num_layers, C = c.num_categories, T = c.time_freq_dim;
  const Layout& L = h->lay;
  const DType mw = c.weight_dtype == GR00T_F32 ? DT_F32 : DT_BF16;
  h->tau.resize(K);
  for (int k = 0; k < K; ++k) h->tau[k] = (int)(((int64_t)c.num_timestep_buckets * k) / K);
  HIPCHK(h, launch_sinusoid(h->tau.data(), K, T, h->w.sin_t, s));
  HIPCHK(h, launch_sinusoid(h->tau.data(), K, D, h->w.tauemb, s));
  // temb = W2 SiLU(W1 sin256(tau) + b1) + b2
  {
    GemmArgs a = ga(h->w.sin_t, T, K, D, T);
    a.W = at<void>(h, L.t_w1);
    a.bias = at<float>(h, L.t_b1);
    HIPCHK(h, launch_gemm_valu(a, ep_store(h->w.t1, true, D, ACT_SILU), DT_F32, mw, s));
    a = ga(h->w.t1, D, K, D, D);
    a.W = at<void>(h, L.t_w2);
    a.bias = at<float>(h, L.t_b2);
    HIPCHK(h, launch_gemm_valu(a, ep_store(h->w.temb, true, D), DT_F32, mw, s));
  }
  HIPCHK(h, launch_silu(h->w.temb, h->w.stemb, (long)K * D, s));
  // [scale | shift] of every block and the output norm: ada[k][l][2D]
  {
    GemmArgs a = ga(h->w.stemb, D, K, (Nl + 1) * 2 * D, D);
    a.W = at<void>(h, L.ada_w);
    a.bias = at<float>(h, L.ada_b);
    HIPCHK(h, launch_gemm_valu(a, ep_store(h->w.ada, true, (long)(Nl + 1) * 2 * D), DT_F32, mw, s));
  }
  // timestep half of the action encoder's second linear, with its bias: c2tab[k][cat][D]
  {
    GemmArgs a = ga(h->w.tauemb, D, K, D, D);
    a.W = at<void>(h, L.ae_w2t);
    a.w_cstride = (long)D * D;
    a.bias = at<float>(h, L.ae_b2);
    a.b_cstride = D;
    a.ids = h->w.iota;
    a.groups = C;
    a.a_gstride = 0;
    Epi e = ep_store(h->w.c2tab, true, (long)C * D);
    e.out_gstride = 0;
    // group g writes columns of category g: offset the output per group via out_row_off
    // is not expressible with a shared row stride, so launch per category.
    for (int cat = 0; cat < C; ++cat) {
      GemmArgs ac = a;
      ac.groups = 1;
      ac.ids = h->w.iota + cat;
      Epi ec = e;
      ec.out = h->w.c2tab + (size_t)cat * D;
      HIPCHK(h, launch_gemm_valu(ac, ec, DT_F32, mw, s));
    }
  }
  return GR00T_OK;
}

// Bytes of the per-sample tables of the training forward for `rows` samples: the sinusoid of
// t, tau's embedding, the two timestep-encoder activations, SiLU(temb), the category term of
// the action encoder and every block's adaLN [scale | shift], each 256-byte aligned.
size_t sample_tables_bytes(const gr00t_config& c, size_t rows) {
  const size_t n[7] = {rows * c.time_freq_dim, rows * c.hidden, rows * c.hidden, rows * c.hidden,
                       rows * c.hidden, rows * c.hidden, rows * (size_t)(c.num_layers + 1) * 2 * c.hidden};
  size_t b = 0;
  for (size_t k : n) b += (k * sizeof(float) + 255) & ~(size_t)255;
  return b;
}

// Per-sample timestep tables of the training forward ("GR00T model class", Flow matching
// diffusion, Training): the bucket floor(t_b * buckets) of each sample, its timestep
// embedding, the adaLN [scale | shift] of every block and of the output norm, and the
// timestep term of the action encoder's second linear under the sample's category. The
// GEMM sequence is that of build_tables with one row per sample instead of one per step.
// The tables go to `base` laid out for `rows` samples (every table fully written, nothing
// accumulated), or, with base NULL, to the handle's own allocation.
int build_sample_tables(gr00t_head* h, const float* t, int B, hipStream_t s, void* base = nullptr, int rows = 0) {
  const gr00t_config& c = h->cfg;
  const int D = c.hidden, Nl = c.num_layers, T = c.time_freq_dim;
  const Layout& L = h->lay;
  const DType mw = c.weight_dtype == GR00T_F32 ? DT_F32 : DT_BF16;
  if (!base) {  // the handle's own tables, sized for max_batch, allocated on the first call
    if (!h->tr_base) {
      if (hipMalloc(&h->tr_base, sample_tables_bytes(c, c.max_batch)) != hipSuccess) {
        h->tr_base = nullptr;
        (void)hipGetLastError();
        return fail(h, GR00T_E_OOM, "training tables: device allocation failed");
      }
    }
    base = h->tr_base;
    rows = c.max_batch;
  }
  const size_t n[7] = {(size_t)rows * T, (size_t)rows * D, (size_t)rows * D, (size_t)rows * D, (size_t)rows * D,
                       (size_t)rows * D, (size_t)rows * (Nl + 1) * 2 * D};
  float** dst[7] = {&h->tr.sin_t, &h->tr.tauemb, &h->tr.t1, &h->tr.temb, &h->tr.stemb, &h->tr.c2, &h->tr.ada};
  char* p = (char*)base;
  for (int i = 0; i < 7; ++i) {
    *dst[i] = (float*)p;
    p += (n[i] * sizeof(float) + 255) & ~(size_t)255;
  }
  HIPCHK(h, launch_sinusoid_t(t, B, c.num_timestep_buckets, T, h->tr.sin_t, s));
  HIPCHK(h, launch_sinusoid_t(t, B, c.num_timestep_buckets, D, h->tr.tauemb, s));
  GemmArgs a = ga(h->tr.sin_t, T, B, D, T);
  a.W = at<void>(h, L.t_w1);
  a.bias = at<float>(h, L.t_b1);
  HIPCHK(h, launch_gemm_valu(a, ep_store(h->tr.t1, true, D, ACT_SILU), DT_F32, mw, s));
  a = ga(h->tr.t1, D, B, D, D);
  a.W = at<void>(h, L.t_w2);
  a.bias = at<float>(h, L.t_b2);
  HIPCHK(h, launch_gemm_valu(a, ep_store(h->tr.temb, true, D), DT_F32, mw, s));
  HIPCHK(h, launch_silu(h->tr.temb, h->tr.stemb, (long)B * D, s));
  a = ga(h->tr.stemb, D, B, (Nl + 1) * 2 * D, D);
  a.W = at<void>(h, L.ada_w);
  a.bias = at<float>(h, L.ada_b);
  HIPCHK(h, launch_gemm_valu(a, ep_store(h->tr.ada, true, (long)(Nl + 1) * 2 * D), DT_F32, mw, s));
  a = ga(h->tr.tauemb, D, 1, D, D);  // one row per sample, the sample's category
  a.groups = B;
  a.a_gstride = 1;
  a.ids = h->w.ids;
  a.W = at<void>(h, L.ae_w2t);
  a.w_cstride = (long)D * D;
  a.bias = at<float>(h, L.ae_b2);
  a.b_cstride = D;
  Epi e = ep_store(h->tr.c2, true, D);
  e.out_gstride = 1;
  HIPCHK(h, launch_gemm_valu(a, e, DT_F32, mw, s));
  return GR00T_OK;
}

// ------------------------------------------------------------------ persistent B = 1 blocks

unsigned* persist_err(gr00t_head* h) {
  PersistArgs pa{};
  persist_bind_scratch(pa, h->persist_base);
  return persist_error_word(pa);
}

// Whether this call's DiT blocks run in the persistent kernel: one sample, bf16 weights and
// activations, the kernel's model widths, and the step graph key's VL length.
bool use_persist(const gr00t_head* h, int B, int L, bool per_sample) {
  const gr00t_config& c = h->cfg;
  return h->persist_ok && B == 1 && !per_sample &&
         persist_b1_fits(c.hidden, c.ff_dim, c.num_heads, c.head_dim, c.action_horizon + 1, L, 256);
}

// Set up the persistent kernel at finalize when the caller asks for it and the model and the
// device allow it.
int persist_setup(gr00t_head* h) {
  const gr00t_config& c = h->cfg;
  int cus = 0;
  HIPCHK(h, hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device));
  if (!(c.flags & GR00T_FLAG_PERSIST) || c.weight_dtype != GR00T_BF16 || c.act_dtype != GR00T_BF16 ||
      !persist_b1_fits(c.hidden, c.ff_dim, c.num_heads, c.head_dim, c.action_horizon + 1, 1, cus))
    return GR00T_OK;
  HIPCHK(h, persist_init());
  const size_t tab = (size_t)c.num_layers * sizeof(PBlock);
  if (hipMalloc(&h->persist_base, persist_scratch_bytes() + tab) != hipSuccess) {
    h->persist_base = nullptr;
    (void)hipGetLastError();
    return fail(h, GR00T_E_OOM, "persistent kernel scratch: device allocation failed");
  }
  HIPCHK(h, hipMemset(h->persist_base, 0, persist_scratch_bytes()));
  h->persist_blocks = (PBlock*)((char*)h->persist_base + persist_scratch_bytes());
  std::vector<PBlock> blocks(c.num_layers);
  for (int l = 0; l < c.num_layers; ++l) {
    const LayerOff& lo = h->lay.L[l];
    PBlock& b = blocks[l];
    b.wq = at<uint16_t>(h, lo.wq);
    b.bq = at<float>(h, lo.bq);
    b.wo = at<uint16_t>(h, lo.wo);
    b.bo = at<float>(h, lo.bo);
    b.w1 = at<uint16_t>(h, lo.w1);
    b.b1 = at<float>(h, lo.b1);
    b.w2 = at<uint16_t>(h, lo.w2);
    b.b2 = at<float>(h, lo.b2);
    b.nq = (l % 2) == 1 ? 3 : 1;
  }
  HIPCHK(h, hipMemcpy(h->persist_blocks, blocks.data(), tab, hipMemcpyHostToDevice));
  h->persist_ok = true;
  return GR00T_OK;
}

// ------------------------------------------------------------------ the launch sequence

// reuse_vl: the VL part (key masks, VL LayerNorm, K/V projection) is skipped and the caches
// of the last full prologue, for the same (B, L_pad), are used as they are.
int run_prologue(gr00t_head* h, const gr00t_inputs* in, hipStream_t s, bool reuse_vl = false) {
  const gr00t_config& c = h->cfg;
  const int B = in->batch, L = in->vl_len, D = c.hidden, E = c.vl_dim, Nc = (c.num_layers + 1) / 2;
  const Layout& lay = h->lay;
  const DType A = h->act;
  const DType mw = c.weight_dtype == GR00T_F32 ? DT_F32 : DT_BF16;
  const DType kvw = (c.weight_dtype == GR00T_FP8_E4M3) ? DT_FP8 : mw;
  LAUNCH(h, s, K_SMALL, launch_sanitize_ids(in->embodiment_id, h->w.ids, h->w.bad, B, c.num_categories, s,
                                            h->w.bad_count));
  if (use_buckets(h, B))
    LAUNCH(h, s, K_SMALL, launch_bucket_ids(h->w.ids, B, c.num_categories, kBucketCap, h->w.perm, h->w.chunks, s));
  if (!reuse_vl) {
    h->kv_B = h->kv_L = 0;  // no valid cache until the projection below is enqueued
    LAUNCH(h, s, K_SMALL, launch_mask_codes(in->vl_mask, in->image_mask, h->w.code, B * L, s));
    // only VL tokens admitted by some block are normalised and projected: their row
    // indices are compacted on the device (vrow[0 .. *vcount))
    LAUNCH(h, s, K_SMALL, launch_compact_rows(h->w.code, B * L, h->w.vrow, h->w.vcount, s));
    LAUNCH(h, s, K_VLLN, launch_layernorm(in->vl_features, A, E, h->w.vln, A, E, B * L, E, at<float>(h, lay.vlln_g),
                                          at<float>(h, lay.vlln_b), nullptr, s, h->w.vrow, h->w.vcount));
    {  // keys and values of every cross block: [valid rows, E] x [Nc*2D, E]^T -> head-major caches
      GemmArgs a = ga(h->w.vln, E, B * L, Nc * 2 * D, E);
      a.rows_dev = h->w.vcount;
      a.W = at<void>(h, lay.kv_w);
      a.bias = at<float>(h, lay.kv_b);
      a.wscale = kvw == DT_FP8 ? at<float>(h, lay.kv_s) : nullptr;
      Epi e{};
      e.kind = EPI_HEADS;
      e.out_f32 = A == DT_F32;
      e.heads[0] = h->w.kc;
      e.heads[1] = h->w.vc;
      e.nwhich = 2;
      e.width = D;
      e.nh = c.num_heads;
      e.hd = c.head_dim;
      e.pos_per_b = L;
      const int Lp = round32(L);
      e.pstride[0] = e.pstride[1] = Lp;
      e.transposed[0] = 0;
      e.transposed[1] = 1;  // values cached [L/32][hd][32] for the attention's V^T operand
      e.layer_stride[0] = e.layer_stride[1] = (long)B * Lp * D;
      e.row_map = h->w.vrow;
      LAUNCH(h, s, K_KV_PROJ, gemm(h, a, e, A, kvw, s));
    }
    h->kv_B = B;
    h->kv_L = L;
  }
  {  // state encoder: one token per sample
    GemmArgs a = ga(in->state, c.state_dim, 1, D, c.state_dim);
    a.groups = B;
    a.a_gstride = 1;
    a.ids = h->w.ids;
    a.W = at<void>(h, lay.se_w1);
    a.w_cstride = (long)D * c.state_dim;
    a.bias = at<float>(h, lay.se_b1);
    a.b_cstride = D;
    Epi e = ep_store(h->w.se1, A == DT_F32, D, ACT_RELU);
    e.out_gstride = 1;
    LAUNCH(h, s, K_STATE_ENC, gemm(h, a, e, DT_F32, mw, s));
    a = ga(h->w.se1, D, 1, D, D);
    a.groups = B;
    a.a_gstride = 1;
    a.ids = h->w.ids;
    a.W = at<void>(h, lay.se_w2);
    a.w_cstride = (long)D * D;
    a.bias = at<float>(h, lay.se_b2);
    a.b_cstride = D;
    e = ep_store(h->w.s, true, D);
    e.out_gstride = 1;
    LAUNCH(h, s, K_STATE_ENC, gemm(h, a, e, A, mw, s));
    if (in->state_features_out)
      LAUNCH(h, s, K_SMALL, launch_copy_rows(h->w.s, D, in->state_features_out, D, 1, 0, B, D, s));
  }
  const long nx = (long)B * c.action_horizon * c.action_dim;
  LAUNCH(h, s, K_SMALL, launch_init_noise(in->noise, h->w.x, nx, c.noise_seed, h->calls, s));
  return GR00T_OK;
}

// Enqueue Euler steps [k0, k1). euler = false writes v of step k0 to w.vout instead.
// per_sample: one forward with every sample's own timestep tables (h->tr: adaLN modulation
// [B][N+1][2D] and the action encoder's timestep term [B][D]) instead of step k0's.
int run_steps(gr00t_head* h, int B, int L, int k0, int k1, bool euler, hipStream_t s, bool per_sample = false) {
  const gr00t_config& c = h->cfg;
  const int D = c.hidden, F = c.ff_dim, H = c.action_horizon, S = H + 1, Adim = c.action_dim, Nl = c.num_layers;
  const int C = c.num_categories, nh = c.num_heads, hd = c.head_dim;
  const Layout& lay = h->lay;
  const DType A = h->act;
  const bool f32 = A == DT_F32;
  const DType mw = c.weight_dtype == GR00T_F32 ? DT_F32 : DT_BF16;
  const DType dw = c.weight_dtype == GR00T_FP8_E4M3 ? DT_FP8 : mw;  // DiT matrices
  const long M = (long)B * S;
  const int Sp = round32(S);
  const size_t ab = act_bytes(h);
  (void)C;
  const int ada_rows = per_sample ? S : 0;
  const long ada_stride = per_sample ? (long)(Nl + 1) * 2 * D : 0;
  for (int k = k0; k < k1; ++k) {
    // [scale | shift] of block l (l = Nl: the output norm)
    auto ada_of = [&](int l) -> const float* {
      return per_sample ? h->tr.ada + (size_t)l * 2 * D : h->w.ada + ((size_t)k * (Nl + 1) + l) * 2 * D;
    };
    // ---- action encoder: a = W1 x + b1; z = swish(W2a a + [W2t tau_emb + b2]); h[1:] = W3 z + b3
    {
      GemmArgs a = ga(h->w.x, Adim, H, D, Adim);
      a.groups = B;
      a.a_gstride = H;
      a.ids = h->w.ids;
      a.W = at<void>(h, lay.ae_w1);
      a.w_cstride = (long)D * Adim;
      a.bias = at<float>(h, lay.ae_b1);
      a.b_cstride = D;
      Epi e = ep_store(h->w.e1, f32, D);
      e.out_gstride = H;
      LAUNCH(h, s, K_ACTION_ENC, gemm(h, a, e, DT_F32, mw, s));
      a = ga(h->w.e1, D, H, D, D);
      a.groups = B;
      a.a_gstride = H;
      a.ids = h->w.ids;
      a.W = at<void>(h, lay.ae_w2a);
      a.w_cstride = (long)D * D;
      e = ep_store(h->w.e2, f32, D, ACT_SILU);
      e.out_gstride = H;
      e.add_tab = per_sample ? h->tr.c2 : h->w.c2tab + (size_t)k * c.num_categories * D;
      e.add_cstride = D;
      e.add_by_group = per_sample ? 1 : 0;
      LAUNCH(h, s, K_ACTION_ENC, gemm(h, a, e, A, mw, s));
      a = ga(h->w.e2, D, H, D, D);
      a.groups = B;
      a.a_gstride = H;
      a.ids = h->w.ids;
      a.W = at<void>(h, lay.ae_w3);
      a.w_cstride = (long)D * D;
      a.bias = at<float>(h, lay.ae_b3);
      a.b_cstride = D;
      e = ep_store(h->w.h, true, D);
      e.out_gstride = S;
      e.out_row_off = 1;
      LAUNCH(h, s, K_ACTION_ENC, gemm(h, a, e, A, mw, s));
      LAUNCH(h, s, K_SMALL, launch_copy_rows(h->w.s, D, h->w.h, D, S, 0, B, D, s));
    }
    // ---- DiT blocks. The two residual GEMMs (o projection, MLP down) may run split-K
    // into fp32 partials; the following norm adds them to h in a fixed order. With at most
    // 32 rows (B = 1) the norm before the MLP is folded into the MLP-up GEMM instead (the
    // skinny kernel normalises the fp32 rows of h as it stages them) and the o projection
    // adds into h directly: one launch fewer per block.
    const bool fold = A == DT_BF16 && dw == DT_BF16 && gemm_ln_fits((int)M, D, dw);
    // W8A8: the LayerNorms before the q / q,k,v, MLP-up and output projections write e4m3 rows
    const bool a8 = use_a8(h, A, dw);
    void* ny = a8 ? (void*)h->w.q8 : h->w.n;
    const DType nt = a8 ? DT_FP8 : A;
    float* nq = a8 ? h->w.qs : nullptr;
    auto normed = [&](int N, const float* ada) {  // A operand of a GEMM that reads LN(h)
      GemmArgs a = ga(fold ? (const void*)h->w.h : (const void*)h->w.n, D, (int)M, N, D);
      if (fold) {
        a.ln = 1;
        a.ln_ada = ada;
      }
      return a;
    };
    int pend = 0;  // partial sums not yet added to h
    const long pstride = M * D;
    if (use_persist(h, B, L, per_sample)) {
      PersistArgs pa{};
      persist_bind_scratch(pa, h->persist_base);
      pa.blocks = h->persist_blocks;
      pa.nl = Nl;
      pa.S = S;
      pa.h = h->w.h;
      pa.ada = ada_of(0);
      pa.kc = (const uint16_t*)h->w.kc;
      pa.vc = (const uint16_t*)h->w.vc;
      pa.Lp = round32(L);
      pa.kv_layer = (long)pa.Lp * D;
      pa.code = h->w.code;
      pa.L = L;
      pa.text_every = c.attend_text_every_n_blocks;
      pa.spin = h->persist_spin;
      LAUNCH(h, s, K_BLOCKS, launch_dit_b1_persist(pa, s));
    }
    for (int l = 0; l < Nl && !use_persist(h, B, L, per_sample); ++l) {
      const LayerOff& lo = lay.L[l];
      const bool self = (l % 2) == 1;
      LAUNCH(h, s, K_ADALN, launch_resid_layernorm(h->w.h, h->w.part, pend, pstride, ny, nt, (int)M, D, ada_of(l), s,
                                                   ada_rows, ada_stride, nq));
      pend = 0;
      {
        GemmArgs a = ga(h->w.n, D, (int)M, (self ? 3 : 1) * D, D);
        a.W = at<void>(h, lo.wq);
        a.bias = at<float>(h, lo.bq);
        a.wscale = dw == DT_FP8 ? at<float>(h, lo.sq) : nullptr;
        Epi e{};
        e.kind = EPI_HEADS;
        e.out_f32 = f32;
        e.heads[0] = h->w.q;
        e.heads[1] = h->w.k;
        e.heads[2] = h->w.v;
        e.nwhich = self ? 3 : 1;
        e.width = D;
        e.nh = nh;
        e.hd = hd;
        e.pos_per_b = S;
        e.pstride[0] = S;
        e.pstride[1] = e.pstride[2] = Sp;
        e.transposed[2] = 1;
        LAUNCH(h, s, self ? K_QKV_PROJ : K_Q_PROJ, a8 ? gemm_q8(h, a, e, s) : gemm(h, a, e, A, dw, s));
      }
      AttnArgs at_{};
      at_.q = h->w.q;
      at_.o = h->w.o;
      at_.B = B;
      at_.S = S;
      at_.nh = nh;
      at_.hd = hd;
      if (self) {
        at_.k = h->w.k;
        at_.vt = h->w.v;
        at_.Lk = S;
        at_.Lp = Sp;
        at_.mask = nullptr;
      } else {
        const size_t ci = (size_t)(l / 2);
        const int Lp = round32(L);
        at_.k = (const char*)h->w.kc + ci * (size_t)B * Lp * D * ab;
        at_.vt = (const char*)h->w.vc + ci * (size_t)B * Lp * D * ab;
        at_.Lk = L;
        at_.Lp = Lp;
        at_.mask = h->w.code;
        at_.mask_bit = (l % (2 * c.attend_text_every_n_blocks) == 0) ? 1 : 2;
      }
      LAUNCH(h, s, self ? K_ATTN_SELF : K_ATTN_CROSS, launch_attention(at_, A, s));
      {
        GemmArgs a = ga(h->w.o, D, (int)M, D, D);
        a.W = at<void>(h, lo.wo);
        a.bias = at<float>(h, lo.bo);
        a.wscale = dw == DT_FP8 ? at<float>(h, lo.so) : nullptr;
        LAUNCH(h, s, K_O_PROJ, resid_gemm(h, a, A, dw, pstride, pend, s, fold));
      }
      if (!fold)
        LAUNCH(h, s, K_NORM3, launch_resid_layernorm(h->w.h, h->w.part, pend, pstride, ny, nt, (int)M, D, nullptr, s, 0, 0, nq));
      pend = 0;
      {
        GemmArgs a = normed(F, nullptr);
        a.W = at<void>(h, lo.w1);
        a.bias = at<float>(h, lo.b1);
        a.wscale = dw == DT_FP8 ? at<float>(h, lo.s1) : nullptr;
        const Epi eu = ep_store(h->w.u, f32, F, ACT_GELU);
        LAUNCH(h, s, K_FF_UP, a8 ? gemm_q8(h, a, eu, s) : gemm(h, a, eu, A, dw, s));
        a = ga(h->w.u, F, (int)M, D, F);
        a.W = at<void>(h, lo.w2);
        a.bias = at<float>(h, lo.b2);
        a.wscale = dw == DT_FP8 ? at<float>(h, lo.s2) : nullptr;
        LAUNCH(h, s, K_FF_DOWN, resid_gemm(h, a, A, dw, pstride, pend, s));
      }
    }
    // ---- output adaLN + projection, then decoder and Euler update
    {
      LAUNCH(h, s, K_ADALN, launch_resid_layernorm(h->w.h, h->w.part, pend, pstride, ny, nt, (int)M, D, ada_of(Nl), s,
                                                   ada_rows, ada_stride, nq));
      GemmArgs a = ga(h->w.n, D, (int)M, D, D);
      a.W = at<void>(h, lay.p_w);
      a.bias = at<float>(h, lay.p_b);
      a.wscale = dw == DT_FP8 ? at<float>(h, lay.p_s) : nullptr;
      const Epi ey = ep_store(h->w.y, f32, D);
      LAUNCH(h, s, K_OUT_PROJ, a8 ? gemm_q8(h, a, ey, s) : gemm(h, a, ey, A, dw, s));
      a = ga(h->w.y, D, H, D, D);
      a.groups = B;
      a.a_gstride = S;
      a.a_row_off = 1;
      a.ids = h->w.ids;
      a.W = at<void>(h, lay.d_w1);
      a.w_cstride = (long)D * D;
      a.bias = at<float>(h, lay.d_b1);
      a.b_cstride = D;
      Epi e = ep_store(h->w.e1, f32, D, ACT_RELU);
      e.out_gstride = H;
      LAUNCH(h, s, K_DECODER, gemm(h, a, e, A, mw, s));
      a = ga(h->w.e1, D, H, Adim, D);
      a.groups = B;
      a.a_gstride = H;
      a.ids = h->w.ids;
      a.W = at<void>(h, lay.d_w2);
      a.w_cstride = (long)Adim * D;
      a.bias = at<float>(h, lay.d_b2);
      a.b_cstride = Adim;
      if (euler) {
        e = ep_store(h->w.x, true, Adim);
        e.kind = EPI_EULER;
        e.dt = 1.0f / (float)c.num_steps;
      } else {
        e = ep_store(h->w.vout, true, Adim);
      }
      e.out_gstride = H;
      LAUNCH(h, s, K_DECODER, gemm(h, a, e, A, mw, s));
    }
  }
  return GR00T_OK;
}

int check_inputs(gr00t_head* h, const gr00t_inputs* in, const void* out, bool reuse_vl = false) {
  if (!h) return GR00T_E_INVALID_ARG;
  if (!in) return fail(h, GR00T_E_INVALID_ARG, "inputs is NULL");
  if (!out) return fail(h, GR00T_E_INVALID_ARG, "output pointer is NULL");
  if (in->batch < 1 || in->batch > h->cfg.max_batch)
    return fail(h, GR00T_E_SHAPE, "batch " + std::to_string(in->batch) + " outside [1, max_batch=" +
                                      std::to_string(h->cfg.max_batch) + "]");
  if (in->vl_len < 1 || in->vl_len > h->cfg.max_vl_len)
    return fail(h, GR00T_E_SHAPE, "vl_len " + std::to_string(in->vl_len) + " outside [1, max_vl_len=" +
                                      std::to_string(h->cfg.max_vl_len) + "]");
  if (!reuse_vl && !in->vl_features) return fail(h, GR00T_E_INVALID_ARG, "vl_features is NULL");
  if (!in->state) return fail(h, GR00T_E_INVALID_ARG, "state is NULL");
  if (!in->embodiment_id) return fail(h, GR00T_E_INVALID_ARG, "embodiment_id is NULL");
  if (!h->finalized) return fail(h, GR00T_E_NOT_FINALIZED, "handle is not finalized");
  if (reuse_vl && (h->kv_B != in->batch || h->kv_L != in->vl_len))
    return fail(h, GR00T_E_NO_VL_CACHE, "no VL key/value cache for (B=" + std::to_string(in->batch) + ", L=" +
                                            std::to_string(in->vl_len) + "): the last full call had (B=" +
                                            std::to_string(h->kv_B) + ", L=" + std::to_string(h->kv_L) + ")");
  return GR00T_OK;
}

// Strict-mode id check on the host, and the deferred report of bad ids seen on the device.
// After a fallback away from a kernel that captured graphs may hold: wait for the device, drop
// every captured graph and capture the prepared step graphs again (whole-call graphs are
// captured anew once their buffers repeat).
int recapture_graphs(gr00t_head* h) {
  if (h->graphs.empty() && h->call_graphs.empty()) return GR00T_OK;
  HIPCHK(h, hipDeviceSynchronize());
  std::vector<std::pair<int, int>> keys;
  for (auto& kv : h->graphs) {
    keys.push_back(kv.first);
    (void)hipGraphExecDestroy(kv.second);
  }
  for (auto& kv : h->call_graphs) (void)hipGraphExecDestroy(kv.second);
  h->graphs.clear();
  h->call_graphs.clear();
  h->call_order.clear();
  h->last_call = CallKey{};
  for (const auto& k : keys) {
    const int rc = gr00t_prepare(h, k.first, k.second);
    if (rc != GR00T_OK) return rc;
  }
  return GR00T_OK;
}

int pre_call_checks(gr00t_head* h, const gr00t_inputs* in, hipStream_t s) {
  uint32_t newest = h->bad_reported, perr = h->persist_err_reported;
  int sample = -1;
  for (auto& r : h->rep) {
    if (!r.recorded || hipEventQuery(r.ev) != hipSuccess) continue;
    uint32_t cnt, pe;
    std::memcpy(&cnt, r.host, 4);
    std::memcpy(&pe, r.host + 4, 4);
    if ((int32_t)(pe - perr) > 0) perr = pe;
    if ((int32_t)(cnt - newest) > 0) {
      newest = cnt;
      sample = -1;
      for (int b = 0; b < r.B && sample < 0; ++b)
        if (r.host[8 + b]) sample = b;
    }
  }
  (void)hipGetLastError();  // a not-ready query leaves no error behind
  if (perr != h->persist_err_reported) {
    h->persist_err_reported = perr;
    h->persist_ok = false;  // later calls take the launch-per-step path, also in the graphs
    const int rc = recapture_graphs(h);
    if (rc != GR00T_OK) return rc;
    return fail(h, GR00T_E_DEVICE_ERROR,
                "an earlier call's persistent block kernel gave up (its workgroups were not all resident at once, or not "
                "32 on each XCD); its result is invalid, and the handle now launches the blocks step by step");
  }
  if (newest != h->bad_reported) {
    const uint32_t n = newest - h->bad_reported;
    h->bad_reported = newest;
    return fail(h, GR00T_E_DEVICE_ERROR,
                "an earlier call met " + std::to_string(n) + " embodiment id(s) outside [0, num_categories)" +
                    (sample >= 0 ? " (sample " + std::to_string(sample) + " of the call whose report was read)" : "") +
                    "; the rows of those samples were set to NaN");
  }
  if (h->cfg.flags & GR00T_FLAG_STRICT) {
    std::vector<int32_t> ids(in->batch);
    HIPCHK(h, hipMemcpyAsync(ids.data(), in->embodiment_id, sizeof(int32_t) * in->batch, hipMemcpyDeviceToHost, s));
    HIPCHK(h, hipStreamSynchronize(s));
    for (int b = 0; b < in->batch; ++b)
      if (ids[b] < 0 || ids[b] >= h->cfg.num_categories)
        return fail(h, GR00T_E_EMBODIMENT, "embodiment_id[" + std::to_string(b) + "] = " + std::to_string(ids[b]) +
                                               " outside [0, " + std::to_string(h->cfg.num_categories) + ")");
  }
  return GR00T_OK;
}

// Enqueue the copy of the invalid-id count and this call's per-sample flags into the next report slot.
int enqueue_report(gr00t_head* h, int B, hipStream_t s) {
  auto& r = h->rep[h->rep_next];
  h->rep_next = (h->rep_next + 1) % gr00t_head::kReportSlots;
  HIPCHK(h, hipMemcpyAsync(r.host, h->w.bad_count, 4, hipMemcpyDeviceToHost, s));
  if (h->persist_ok) HIPCHK(h, hipMemcpyAsync(r.host + 4, persist_err(h), 4, hipMemcpyDeviceToHost, s));
  HIPCHK(h, hipMemcpyAsync(r.host + 8, h->w.bad, B, hipMemcpyDeviceToHost, s));
  HIPCHK(h, hipEventRecord(r.ev, s));
  r.recorded = true;
  r.B = B;
  return GR00T_OK;
}

}  // namespace

namespace {
int train_forward(gr00t_head* h, const gr00t_inputs* in, const float* actions, const float* t, float* loss,
                  float* v_pred, void* hip_stream, bool no_alloc) {
  int rc = check_inputs(h, in, loss);
  if (rc != GR00T_OK) return rc;
  if (!actions || !t) return fail(h, GR00T_E_INVALID_ARG, "actions and t are required");
  if (!in->noise) return fail(h, GR00T_E_INVALID_ARG, "the training forward needs inputs.noise");
  const gr00t_config& c = h->cfg;
  const int B = in->batch, per = c.action_horizon * c.action_dim;
  if (no_alloc) {
    const size_t need = sample_tables_bytes(c, B);
    if (need > static_scratch_bytes())
      return fail(h, GR00T_E_SHAPE,
                  "gr00t_train_forward_noalloc: " + std::to_string(B) + " samples need " + std::to_string(need) +
                      " bytes of per-sample tables; the fixed scratch area holds " +
                      std::to_string(static_scratch_bytes()) + " (" +
                      std::to_string(static_scratch_bytes() / sample_tables_bytes(c, 1)) + " samples of this model)");
  }
  hipStream_t s = (hipStream_t)hip_stream;
  HIPCHK(h, hipSetDevice(h->device));
  rc = pre_call_checks(h, in, s);
  if (rc != GR00T_OK) return rc;
  rc = run_prologue(h, in, s);  // VL, ids, state token (its x = noise is replaced below)
  if (rc != GR00T_OK) return rc;
  rc = no_alloc ? build_sample_tables(h, t, B, s, h->static_scratch, B) : build_sample_tables(h, t, B, s);
  if (rc != GR00T_OK) return rc;
  LAUNCH(h, s, K_SMALL, launch_flow_interp(actions, in->noise, t, h->w.x, B, per, s));
  rc = run_steps(h, B, in->vl_len, 0, 1, false, s, true);
  if (rc != GR00T_OK) return rc;
  LAUNCH(h, s, K_SMALL, launch_masked_mse(h->w.vout, actions, in->noise, in->action_mask, h->w.bad, B, per, loss, s));
  if (v_pred) HIPCHK(h, hipMemcpyAsync(v_pred, h->w.vout, sizeof(float) * B * per, hipMemcpyDeviceToDevice, s));
  rc = enqueue_report(h, B, s);
  if (rc != GR00T_OK) return rc;
  h->calls++;
  return GR00T_OK;
}
}  // namespace

// ====================================================================== C ABI

extern "C" {

int gr00t_create(const gr00t_config* cfg, int device, gr00t_head** out) {
  g_create_error.clear();
  if (!out) {
    g_create_error = "out is NULL";
    return GR00T_E_INVALID_ARG;
  }
  *out = nullptr;
  std::string why;
  int rc = check_config(cfg, why);
  if (rc != GR00T_OK) {
    g_create_error = why;
    return rc;
  }
  if (device < 0) {
    g_create_error = "device must be >= 0";
    return GR00T_E_INVALID_ARG;
  }
  gr00t_head* h = new (std::nothrow) gr00t_head();
  if (!h) {
    g_create_error = "out of host memory";
    return GR00T_E_OOM;
  }
  h->cfg = *cfg;
  if (const char* sp = std::getenv("GR00T_PERSIST_SPIN")) h->persist_spin = (unsigned)std::strtoul(sp, nullptr, 10);
  h->device = device;
  h->act = cfg->act_dtype == GR00T_F32 ? DT_F32 : DT_BF16;
  build_specs(h);
  *out = h;
  return GR00T_OK;
}

int gr00t_load_weights(gr00t_head* h, const char* name, const void* host_data, gr00t_dtype dtype,
                       const int64_t* shape, int ndim) {
  if (!h) return GR00T_E_INVALID_ARG;
  if (h->finalized) return fail(h, GR00T_E_NOT_FINALIZED, "weights cannot be loaded after finalize");
  if (!name || !host_data || (!shape && ndim > 0) || ndim < 0)
    return fail(h, GR00T_E_INVALID_ARG, "name, host_data and shape must be non-NULL");
  auto it = h->specs.find(name);
  if (it == h->specs.end()) return fail(h, GR00T_E_UNKNOWN_WEIGHT, std::string("unknown weight '") + name + "'");
  Spec& s = it->second;
  std::vector<int64_t> got(shape, shape + ndim);
  if (got != s.shape)
    return fail(h, GR00T_E_SHAPE, std::string("weight '") + name + "' has shape " + shape_str(got) + ", expected " +
                                      shape_str(s.shape));
  if (dtype != GR00T_F32 && dtype != GR00T_BF16)
    return fail(h, GR00T_E_INVALID_ARG, std::string("weight '") + name + "': dtype must be F32 or BF16");
  if (dtype == GR00T_BF16 && s.store != ST_BF16)
    return fail(h, GR00T_E_INVALID_ARG, std::string("weight '") + name +
                                            "': BF16 input is accepted only for tensors stored as bf16 matrices");
  try {
    pack(h, s, host_data, dtype);
  } catch (const std::bad_alloc&) {
    return fail(h, GR00T_E_OOM, "out of host memory while packing '" + std::string(name) + "'");
  }
  s.loaded = true;
  return GR00T_OK;
}

int gr00t_finalize(gr00t_head* h) {
  if (!h) return GR00T_E_INVALID_ARG;
  if (h->finalized) return GR00T_OK;
  for (const std::string& n : h->order)
    if (!h->specs[n].loaded) return fail(h, GR00T_E_MISSING_WEIGHT, "weight '" + n + "' was never loaded");
  const gr00t_config& c = h->cfg;
  HIPCHK(h, hipSetDevice(h->device));
  if (hipMalloc((void**)&h->arena, h->lay.total) != hipSuccess) {
    h->arena = nullptr;
    (void)hipGetLastError();
    return fail(h, GR00T_E_OOM, "hipMalloc of " + std::to_string(h->lay.total) + " weight bytes failed");
  }
  for (const std::string& n : h->order) {
    Spec& s = h->specs[n];
    size_t pos = 0;
    for (const Piece& p : s.pieces) {
      if (!s.matrix) {
        HIPCHK(h, hipMemcpy(h->arena + p.off, s.staged.data(), s.staged.size(), hipMemcpyHostToDevice));
        pos = s.staged.size();
        continue;
      }
      const size_t nd = s.shape.size();
      const size_t C = nd == 3 ? s.shape[0] : 1, OUT = s.shape[nd - 1];
      const size_t esz = s.store == ST_F32 ? 4 : (s.store == ST_BF16 ? 2 : 1);
      const size_t bytes = C * OUT * p.in_n * esz;
      HIPCHK(h, hipMemcpy(h->arena + p.off, s.staged.data() + pos, bytes, hipMemcpyHostToDevice));
      pos += bytes;
      if (s.store == ST_FP8) {
        HIPCHK(h, hipMemcpy(h->arena + p.scale_off, s.staged.data() + pos, C * OUT * 4, hipMemcpyHostToDevice));
        pos += C * OUT * 4;
      }
    }
    std::vector<uint8_t>().swap(s.staged);
  }
  // workspace
  const size_t Bm = c.max_batch, Lm = c.max_vl_len, D = c.hidden, F = c.ff_dim, H = c.action_horizon, S = H + 1;
  const size_t A = c.action_dim, E = c.vl_dim, K = c.num_steps, Nl = c.num_layers, Nc = (Nl + 1) / 2;
  const size_t C = c.num_categories, T = c.time_freq_dim;
  const size_t Sp = round32((int)S), Lmp = round32((int)Lm);
  const size_t ab = act_bytes(h);
  const bool w8a8 = (c.flags & GR00T_FLAG_W8A8) != 0;
  std::vector<std::pair<void**, size_t>> req = {
      {(void**)&h->w.h, Bm * S * D * 4},      {&h->w.n, Bm * S * D * ab},       {&h->w.q, Bm * S * D * ab},
      {&h->w.k, Bm * Sp * D * ab},            {&h->w.v, Bm * Sp * D * ab},      {&h->w.o, Bm * S * D * ab},
      {&h->w.u, Bm * S * F * ab},             {&h->w.y, Bm * S * D * ab},       {&h->w.e1, Bm * H * D * ab},
      {&h->w.e2, Bm * H * D * ab},            {&h->w.se1, Bm * D * ab},         {&h->w.vln, Bm * Lm * E * ab},
      {&h->w.kc, Nc * Bm * Lmp * D * ab},     {&h->w.vc, Nc * Bm * Lmp * D * ab}, {(void**)&h->w.x, Bm * H * A * 4},
      {(void**)&h->w.s, Bm * D * 4},          {(void**)&h->w.vout, Bm * H * A * 4},
      {(void**)&h->w.part, 8 * Bm * S * D * 4},
      {(void**)&h->w.code, Bm * Lm},          {(void**)&h->w.bad, Bm},           {(void**)&h->w.ids, Bm * 4},
      {(void**)&h->w.bad_count, 4},
      {(void**)&h->w.vrow, Bm * Lm * 4},      {(void**)&h->w.vcount, 4},
      {(void**)&h->w.iota, C * 4},            {(void**)&h->w.sin_t, K * T * 4},  {(void**)&h->w.t1, K * D * 4},
      {(void**)&h->w.temb, K * D * 4},        {(void**)&h->w.stemb, K * D * 4},
      {(void**)&h->w.ada, K * (Nl + 1) * 2 * D * 4},                              {(void**)&h->w.tauemb, K * D * 4},
      {(void**)&h->w.c2tab, K * C * D * 4},
      {(void**)&h->w.q8, w8a8 ? std::max(Bm * Lm * E, Bm * S * std::max(F, D)) : 0},
      {(void**)&h->w.qs, w8a8 ? std::max(Bm * Lm, Bm * S) * 4 : 0},
      {(void**)&h->w.perm, Bm * 4},
      {(void**)&h->w.chunks, (size_t)bucket_max_chunks((int)Bm, (int)C, kBucketCap) * sizeof(int4)}};
  size_t total = 0;
  for (auto& r : req) total += (r.second + 255) & ~(size_t)255;
  if (hipMalloc((void**)&h->wsbase, total) != hipSuccess) {
    h->wsbase = nullptr;
    (void)hipGetLastError();
    return fail(h, GR00T_E_OOM, "hipMalloc of " + std::to_string(total) + " workspace bytes failed");
  }
  h->ws_bytes = total;
  size_t off = 0;
  for (auto& r : req) {
    *r.first = h->wsbase + off;
    off += (r.second + 255) & ~(size_t)255;
  }
  std::vector<int> iota(C);
  for (size_t i = 0; i < C; ++i) iota[i] = (int)i;
  HIPCHK(h, hipMemcpy(h->w.iota, iota.data(), C * 4, hipMemcpyHostToDevice));
  HIPCHK(h, hipMemset(h->w.bad, 0, Bm));
  HIPCHK(h, hipMemset(h->w.bad_count, 0, 4));
  // key/value padding rows and columns are read with weight 0: keep them finite
  HIPCHK(h, hipMemset(h->w.kc, 0, Nc * Bm * Lmp * D * ab));
  HIPCHK(h, hipMemset(h->w.vc, 0, Nc * Bm * Lmp * D * ab));
  HIPCHK(h, hipMemset(h->w.k, 0, Bm * Sp * D * ab));
  HIPCHK(h, hipMemset(h->w.v, 0, Bm * Sp * D * ab));
  HIPCHK(h, hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  for (auto& r : h->rep) {
    HIPCHK(h, hipHostMalloc((void**)&r.host, 8 + Bm, hipHostMallocDefault));
    std::memset(r.host, 0, 8 + Bm);
    HIPCHK(h, hipEventCreateWithFlags(&r.ev, hipEventDisableTiming));
  }
  HIPCHK(h, static_scratch_address(h->device, &h->static_scratch));
  int rc = persist_setup(h);
  if (rc != GR00T_OK) return rc;
  rc = build_tables(h, h->cap_stream);
  if (rc != GR00T_OK) return rc;
  HIPCHK(h, hipStreamSynchronize(h->cap_stream));
  h->finalized = true;
  return GR00T_OK;
}

int gr00t_prepare(gr00t_head* h, int32_t batch, int32_t vl_len) {
  if (!h) return GR00T_E_INVALID_ARG;
  if (!h->finalized) return fail(h, GR00T_E_NOT_FINALIZED, "handle is not finalized");
  if (!(h->cfg.flags & GR00T_FLAG_USE_GRAPH)) return fail(h, GR00T_E_INVALID_ARG, "prepare needs GR00T_FLAG_USE_GRAPH");
  if (batch < 1 || batch > h->cfg.max_batch || vl_len < 1 || vl_len > h->cfg.max_vl_len)
    return fail(h, GR00T_E_SHAPE, "prepare shape outside capacity");
  const auto key = std::make_pair((int)batch, (int)vl_len);
  if (h->graphs.count(key)) return GR00T_OK;
  HIPCHK(h, hipSetDevice(h->device));
  hipGraph_t g = nullptr;
  HIPCHK(h, hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  const bool prof = h->prof_on;
  h->prof_on = false;  // no event records inside the graph
  int rc = run_steps(h, batch, vl_len, 0, h->cfg.num_steps, true, h->cap_stream);
  h->prof_on = prof;
  hipError_t e = hipStreamEndCapture(h->cap_stream, &g);
  if (rc != GR00T_OK) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(h, GR00T_E_HIP, std::string("hipStreamEndCapture failed: ") + hipGetErrorString(e));
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return fail(h, GR00T_E_HIP, std::string("hipGraphInstantiate failed: ") + hipGetErrorString(e));
  h->graphs[key] = ex;
  return GR00T_OK;
}

// Capture prologue, K steps and output of a call with these buffers as one graph (evicting the
// oldest of kMaxCallGraphs; the device is synchronised first, as the evicted graph may still run).
static int capture_call(gr00t_head* h, const gr00t_inputs* in, float* action_pred, const CallKey& k) {
  if (h->call_graphs.size() >= kMaxCallGraphs) {
    HIPCHK(h, hipDeviceSynchronize());
    (void)hipGraphExecDestroy(h->call_graphs[h->call_order.front()]);
    h->call_graphs.erase(h->call_order.front());
    h->call_order.erase(h->call_order.begin());
  }
  const int kv_B = h->kv_B, kv_L = h->kv_L;
  hipGraph_t g = nullptr;
  HIPCHK(h, hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  const bool prof = h->prof_on;
  h->prof_on = false;  // no event records inside the graph
  int rc = run_prologue(h, in, h->cap_stream, false);
  if (rc == GR00T_OK) rc = run_steps(h, in->batch, in->vl_len, 0, h->cfg.num_steps, true, h->cap_stream);
  hipError_t e = hipSuccess;
  if (rc == GR00T_OK)
    e = launch_output(h->w.x, in->action_mask, h->w.bad, action_pred, in->batch,
                      h->cfg.action_horizon * h->cfg.action_dim, h->cap_stream);
  h->prof_on = prof;
  h->kv_B = kv_B;  // nothing ran yet: the caches are those of before
  h->kv_L = kv_L;
  hipError_t ee = hipStreamEndCapture(h->cap_stream, &g);
  if (rc != GR00T_OK || e != hipSuccess || ee != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    if (rc != GR00T_OK) return rc;
    return fail(h, GR00T_E_HIP, std::string("whole-call capture failed: ") + hipGetErrorString(e != hipSuccess ? e : ee));
  }
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (e != hipSuccess) return fail(h, GR00T_E_HIP, std::string("hipGraphInstantiate failed: ") + hipGetErrorString(e));
  h->call_graphs[k] = ex;
  h->call_order.push_back(k);
  return GR00T_OK;
}

static int get_action(gr00t_head* h, const gr00t_inputs* in, float* action_pred, void* hip_stream, bool reuse_vl) {
  int rc = check_inputs(h, in, action_pred, reuse_vl);
  if (rc != GR00T_OK) return rc;
  const bool use_graph = (h->cfg.flags & GR00T_FLAG_USE_GRAPH) != 0;
  const auto key = std::make_pair((int)in->batch, (int)in->vl_len);
  const bool have_graph = use_graph && h->graphs.count(key) && !(h->prof_on && h->prof_mode == 1);
  if (use_graph && !have_graph && (h->cfg.flags & GR00T_FLAG_STRICT))
    return fail(h, GR00T_E_UNCAPTURED, "shape (B=" + std::to_string(in->batch) + ", L=" + std::to_string(in->vl_len) +
                                           ") was not prepared");
  hipStream_t s = (hipStream_t)hip_stream;
  HIPCHK(h, hipSetDevice(h->device));
  rc = pre_call_checks(h, in, s);
  if (rc != GR00T_OK) return rc;
  // A full call with caller noise on a prepared shape whose buffers repeat those of the previous
  // call replays one graph of the whole call (captured on that repetition).
  if (have_graph && !reuse_vl && in->noise) {
    CallKey k;
    k.B = in->batch;
    k.L = in->vl_len;
    k.p = {in->vl_features, in->vl_mask, in->image_mask, in->state, in->embodiment_id, in->noise, in->action_mask,
           in->state_features_out, action_pred};
    auto it = h->call_graphs.find(k);
    if (it == h->call_graphs.end() && k == h->last_call) {
      rc = capture_call(h, in, action_pred, k);
      if (rc != GR00T_OK) return rc;
      it = h->call_graphs.find(k);
    }
    h->last_call = k;
    if (it != h->call_graphs.end()) {
      LAUNCH(h, s, K_CALL_GRAPH, hipGraphLaunch(it->second, s));
      h->kv_B = in->batch;  // the replayed prologue rebuilt the VL key/value caches
      h->kv_L = in->vl_len;
      rc = enqueue_report(h, in->batch, s);
      if (rc != GR00T_OK) return rc;
      h->calls++;
      return GR00T_OK;
    }
  }
  rc = run_prologue(h, in, s, reuse_vl);
  if (rc != GR00T_OK) return rc;
  if (have_graph) {
    LAUNCH(h, s, K_GRAPH, hipGraphLaunch(h->graphs[key], s));
  } else {
    rc = run_steps(h, in->batch, in->vl_len, 0, h->cfg.num_steps, true, s);
    if (rc != GR00T_OK) return rc;
  }
  LAUNCH(h, s, K_SMALL, launch_output(h->w.x, in->action_mask, h->w.bad, action_pred, in->batch,
                          h->cfg.action_horizon * h->cfg.action_dim, s));
  rc = enqueue_report(h, in->batch, s);
  if (rc != GR00T_OK) return rc;
  h->calls++;
  return GR00T_OK;
}

int gr00t_get_action(gr00t_head* h, const gr00t_inputs* in, float* action_pred, void* hip_stream) {
  return get_action(h, in, action_pred, hip_stream, false);
}

int gr00t_get_action_reuse_vl(gr00t_head* h, const gr00t_inputs* in, float* action_pred, void* hip_stream) {
  return get_action(h, in, action_pred, hip_stream, true);
}


int gr00t_train_forward(gr00t_head* h, const gr00t_inputs* in, const float* actions, const float* t, float* loss,
                        float* v_pred, void* hip_stream) {
  return train_forward(h, in, actions, t, loss, v_pred, hip_stream, false);
}

int gr00t_train_forward_noalloc(gr00t_head* h, const gr00t_inputs* in, const float* actions, const float* t,
                                float* loss, float* v_pred, void* hip_stream) {
  return train_forward(h, in, actions, t, loss, v_pred, hip_stream, true);
}

#ifdef GR00T_PHASE_TRACE
// Diagnostic builds only (flow_matching_dit_amd/phase_trace.py): copy the persistent kernel's
// phase timestamps of its last launch (persist_trace_words() values, s_memrealtime at 100 MHz)
// to the host. Synchronous.
int gr00t_persist_phase_trace(gr00t_head* h, uint64_t* host, int32_t n) {
  if (!h || !host || n < persist_trace_words()) return GR00T_E_INVALID_ARG;
  if (!h->persist_base) return fail(h, GR00T_E_INVALID_ARG, "the handle has no persistent kernel");
  PersistArgs pa{};
  persist_bind_scratch(pa, h->persist_base);
  HIPCHK(h, hipSetDevice(h->device));
  HIPCHK(h, hipDeviceSynchronize());
  HIPCHK(h, hipMemcpy(host, pa.trace, sizeof(uint64_t) * persist_trace_words(), hipMemcpyDeviceToHost));
  return GR00T_OK;
}
#endif

int gr00t_velocity(gr00t_head* h, const gr00t_inputs* in, int32_t step_k, float* v, void* hip_stream) {
  int rc = check_inputs(h, in, v);
  if (rc != GR00T_OK) return rc;
  if (!in->noise) return fail(h, GR00T_E_INVALID_ARG, "gr00t_velocity needs inputs.noise");
  if (step_k < 0 || step_k >= h->cfg.num_steps) return fail(h, GR00T_E_INVALID_ARG, "step_k outside [0, num_steps)");
  hipStream_t s = (hipStream_t)hip_stream;
  HIPCHK(h, hipSetDevice(h->device));
  rc = pre_call_checks(h, in, s);
  if (rc != GR00T_OK) return rc;
  rc = run_prologue(h, in, s);
  if (rc != GR00T_OK) return rc;
  rc = run_steps(h, in->batch, in->vl_len, step_k, step_k + 1, false, s);
  if (rc != GR00T_OK) return rc;
  HIPCHK(h, hipMemcpyAsync(v, h->w.vout, sizeof(float) * in->batch * h->cfg.action_horizon * h->cfg.action_dim,
                           hipMemcpyDeviceToDevice, s));
  h->calls++;
  return GR00T_OK;
}

int gr00t_quantize_e4m3_rows(gr00t_head* h, const void* x, int64_t ld_x, int32_t rows, int32_t cols, uint8_t* q,
                             float* scale, void* hip_stream) {
  if (!h) return GR00T_E_INVALID_ARG;
  if (!x || !q || !scale) return fail(h, GR00T_E_INVALID_ARG, "gr00t_quantize_e4m3_rows: NULL pointer");
  if (((uintptr_t)x % 16) || ((uintptr_t)q % 8) || ((uintptr_t)scale % 4))
    return fail(h, GR00T_E_INVALID_ARG, "gr00t_quantize_e4m3_rows: x must be 16-byte, q 8-byte aligned");
  if (rows < 0 || cols < 8 || cols % 8 || ld_x < cols || ld_x % 8)
    return fail(h, GR00T_E_INVALID_ARG,
                "gr00t_quantize_e4m3_rows: needs rows >= 0, cols a positive multiple of 8, ld_x >= cols and a "
                "multiple of 8");
  if (rows == 0) return GR00T_OK;
  HIPCHK(h, hipSetDevice(h->device));
  HIPCHK(h, launch_quant_rows(x, ld_x, rows, cols, q, cols, scale, (hipStream_t)hip_stream));
  return GR00T_OK;
}

void gr00t_destroy(gr00t_head* h) {
  if (!h) return;
  if (h->finalized || h->arena || h->wsbase) {
    (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();  // copies into the pinned report slots may still be in flight
  }
  for (auto& kv : h->graphs) (void)hipGraphExecDestroy(kv.second);
  for (auto& kv : h->call_graphs) (void)hipGraphExecDestroy(kv.second);
  if (h->cap_stream) {
    (void)hipStreamSynchronize(h->cap_stream);
    (void)hipStreamDestroy(h->cap_stream);
  }
  for (auto& r : h->rep) {
    if (r.ev) (void)hipEventDestroy(r.ev);
    if (r.host) (void)hipHostFree(r.host);
  }
  for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
  if (h->tr_base) (void)hipFree(h->tr_base);
  if (h->persist_base) (void)hipFree(h->persist_base);
  if (h->arena || h->wsbase) (void)hipDeviceSynchronize();
  if (h->arena) (void)hipFree(h->arena);
  if (h->wsbase) (void)hipFree(h->wsbase);
  delete h;
}

int gr00t_profile_enable(gr00t_head* h, int on) {
  if (!h) return GR00T_E_INVALID_ARG;
  if (h->prof_on) {
    int rc = prof_collect(h);
    if (rc != GR00T_OK) return rc;
  }
  if (on < 0 || on > 2) return fail(h, GR00T_E_INVALID_ARG, "profiling mode must be 0, 1 or 2");
  h->prof_on = on != 0;
  h->prof_mode = on;
  h->prof_n.assign(K_NCLASS, 0);
  h->prof_ms.assign(K_NCLASS, 0.0);
  return GR00T_OK;
}

int gr00t_profile_read(gr00t_head* h, int kclass, int64_t* launches, double* total_ms) {
  if (!h || !launches || !total_ms) return GR00T_E_INVALID_ARG;
  if (kclass < 0 || kclass >= K_NCLASS) return fail(h, GR00T_E_INVALID_ARG, "kclass out of range");
  if (h->prof_n.empty()) {
    h->prof_n.assign(K_NCLASS, 0);
    h->prof_ms.assign(K_NCLASS, 0.0);
  }
  int rc = prof_collect(h);
  if (rc != GR00T_OK) return rc;
  *launches = h->prof_n[kclass];
  *total_ms = h->prof_ms[kclass];
  return GR00T_OK;
}

const char* gr00t_profile_class_name(int kclass) {
  if (kclass < 0 || kclass >= K_NCLASS) return nullptr;
  return kClassNames[kclass];
}

const char* gr00t_last_error(const gr00t_head* h) {
  if (!h) return g_create_error.c_str();
  return h->err.c_str();
}

size_t gr00t_device_bytes(const gr00t_head* h) {
  if (!h || !h->finalized) return 0;
  return h->lay.total + h->ws_bytes;
}

}  // extern "C"

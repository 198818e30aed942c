/*
 * gr00t_head.h -- C ABI of the MI355X (gfx950) GR00T flow-matching DiT action head.
 *
 * The head is System 1 of the GR00T vision-language-action model ("Model
 * architecture" page, sections "Action head architecture", "Diffusion
 * transformer (DiT)", "AlternateVLDiT variant", "Flow matching diffusion" and
 * "Embodiment-specific projectors"; "GR00T model class" page, section
 * "get_action"). Given backbone features [B, L, 2048] with their attention and
 * image masks, the robot state and an embodiment id per sample, it integrates
 * K Euler steps  x <- x + (1/K) * v(x, tau_k)  of a DiT velocity field starting
 * from Gaussian noise and returns action_pred [B, H, A].
 *
 * Conventions for every entry point:
 *   - Return value: GR00T_OK (0) or a negative gr00t_status. No C++ exception
 *     crosses this boundary. The message of the last failure on a handle is
 *     returned by gr00t_last_error(handle).
 *   - Every argument check runs before any device work is enqueued.
 *   - "device" pointers point to memory on the handle's GPU; "host" pointers to
 *     ordinary host memory. The caller owns every buffer it passes and keeps it
 *     valid until the work on the given stream has completed.
 *   - One call may be in flight per handle at a time; distinct handles are
 *     independent.
 */
#ifndef GR00T_HEAD_H
#define GR00T_HEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gr00t_status {
  GR00T_OK = 0,
  GR00T_E_INVALID_ARG = -1,    /* NULL handle/pointer, bad enum, inconsistent config */
  GR00T_E_SHAPE = -2,          /* B > max_batch, L_pad > max_vl_len, weight shape mismatch */
  GR00T_E_EMBODIMENT = -3,     /* strict mode: an embodiment id outside [0, num_categories) */
  GR00T_E_NOT_FINALIZED = -4,  /* get_action/prepare before finalize, or load after it */
  GR00T_E_UNKNOWN_WEIGHT = -5, /* load_weights with a name the config does not define */
  GR00T_E_UNCAPTURED = -6,     /* USE_GRAPH|STRICT and (B, L_pad) was not prepared */
  GR00T_E_HIP = -7,            /* a HIP runtime call failed (message names it) */
  GR00T_E_OOM = -8,            /* device allocation failed */
  GR00T_E_MISSING_WEIGHT = -9, /* finalize with a weight never loaded */
  GR00T_E_DEVICE_ERROR = -10,  /* a previous call met an invalid id in non-strict mode */
  GR00T_E_NO_VL_CACHE = -11    /* reuse_vl call without a full call of the same (B, L_pad) */
} gr00t_status;

typedef enum gr00t_dtype {
  GR00T_F32 = 0,
  GR00T_BF16 = 1,
  GR00T_FP8_E4M3 = 2, /* OCP E4M3 ("fn": no inf, max 448) */
  GR00T_U8 = 3,
  GR00T_I32 = 4
} gr00t_dtype;

/* Flags of gr00t_config.flags. */
#define GR00T_FLAG_STRICT 0x1u    /* the Policy API's `strict` validation ("Understanding the
                                     GR00T Policy API", Loading the Policy: observation shapes
                                     and dtypes checked at run time, at a cost in speed): ids
                                     are copied to the host and checked (E_EMBODIMENT) and, in
                                     graph mode, an unprepared shape is refused (E_UNCAPTURED).
                                     Shapes and dtypes of the tensors behind the pointers are
                                     checked by the Python binding, which knows them. */
#define GR00T_FLAG_USE_GRAPH 0x2u /* replay the K-step loop from a captured hipGraph (see
                                     gr00t_prepare); a gr00t_get_action on a prepared shape
                                     with inputs.noise given, whose buffers (every pointer of
                                     gr00t_inputs and action_pred) are those of the previous
                                     call, is captured as one graph of the whole call (prologue,
                                     K steps, output) and replayed whenever those buffers come
                                     again; up to 8 such graphs per handle, the oldest evicted
                                     (the device is synchronised first). Buffer contents are read
                                     at each replay; a buffer freed and reallocated at the same
                                     address is simply reused. */
#define GR00T_FLAG_W8A8 0x4u      /* with FP8_E4M3 weights: the input rows of every e4m3-weight
                                     GEMM (the DiT's q, k, v, o, MLP and output projections and
                                     the VL key/value projection) are quantised to e4m3 with one
                                     fp32 scale per row (amax / 448) and multiplied on the fp8
                                     matrix cores; FP8 weights required, else GR00T_E_INVALID_ARG
                                     at create. Adds K + 4 bytes per row of the largest such
                                     GEMM input to the workspace. */

#define GR00T_FLAG_PERSIST 0x8u /* run the DiT blocks of a one-sample call (bf16, hidden 1536,
                                   32 heads of 48, MLP 6144, at most 32 tokens) in one persistent
                                   kernel per Euler step, one workgroup per compute unit that
                                   streams each block's weights while it waits for the others,
                                   instead of one launch per step of the block. The kernel needs
                                   all 256 compute units to itself: a wait that does not end
                                   within its bound gives up, the call's result is then wrong,
                                   the next call reports GR00T_E_DEVICE and the handle falls back
                                   to the launch-per-step path (its captured graphs are captured
                                   again). Ignored where it does not apply. The environment
                                   variable GR00T_PERSIST_SPIN, read at gr00t_create, sets how
                                   many polls a wait makes before it gives up (tests of the
                                   fallback; default 2^20). */

#define GR00T_FLAG_NO_BUCKETS 0x10u /* batches of 128 samples or more normally run the
                                       per-embodiment bf16 linears over category buckets (the
                                       samples sorted by embodiment id on the device, each
                                       category's weights read once per bucket of up to 8
                                       samples; "Model architecture", Embodiment-specific
                                       projectors, CategorySpecificLinear: W[cat_ids] then a
                                       batched product). With this flag every sample gathers its
                                       own category's weights, as for smaller batches; for
                                       comparison */

/*
 * Model and capacity. Widths follow the "Model configuration" table of the
 * architecture page: hidden = num_heads * head_dim is used for the state and
 * action encoders' output, the DiT inner width and the decoder's hidden width.
 */
typedef struct gr00t_config {
  int32_t num_layers;        /* DiT blocks; even index = cross-attention, odd = self */
  int32_t hidden;            /* D */
  int32_t num_heads;
  int32_t head_dim;          /* D == num_heads * head_dim; head_dim <= 64, multiple of 16 */
  int32_t ff_dim;            /* F, GELU MLP width */
  int32_t vl_dim;            /* backbone_embedding_dim (2048 on the pages) */
  int32_t state_dim;         /* state features per sample (one state token) */
  int32_t action_dim;        /* A */
  int32_t action_horizon;    /* H; the DiT sees S = 1 + H tokens */
  int32_t num_categories;    /* C, embodiment tables */
  int32_t num_steps;         /* K Euler steps (num_inference_timesteps) */
  int32_t num_timestep_buckets;       /* 1000 */
  int32_t attend_text_every_n_blocks; /* n of the AlternateVLDiT text/image alternation */
  int32_t time_freq_dim;     /* width of the timestep sinusoid fed to the timestep encoder */
  int32_t max_batch;         /* capacity: largest B served */
  int32_t max_vl_len;        /* capacity: largest L_pad served */
  gr00t_dtype weight_dtype;  /* F32, BF16 or FP8_E4M3 (e4m3 DiT matrices, the rest bf16) */
  gr00t_dtype act_dtype;     /* F32 (with F32 weights) or BF16 */
  uint32_t flags;            /* GR00T_FLAG_* */
  uint64_t noise_seed;       /* seed of the library's N(0,1) draw when inputs.noise == NULL */
} gr00t_config;

/*
 * Inputs of one get_action call ("GR00T model class", get_action; the backbone
 * output dict of the architecture page: backbone_features, backbone_attention_mask,
 * image_mask). All pointers are device pointers unless noted.
 */
typedef struct gr00t_inputs {
  int32_t batch;                 /* B (host value), 1 <= B <= max_batch */
  int32_t vl_len;                /* L_pad (host value), 1 <= L_pad <= max_vl_len */
  const void* vl_features;       /* [B, L_pad, vl_dim] in act_dtype, row-major */
  const uint8_t* vl_mask;        /* [B, L_pad] 0/1, NULL = every position valid */
  const uint8_t* image_mask;     /* [B, L_pad] 0/1, NULL = no image/text split: every
                                    cross block attends to all valid positions */
  const float* state;            /* [B, 1, state_dim] f32 */
  const int32_t* embodiment_id;  /* [B] in [0, num_categories) */
  const float* noise;            /* [B, H, A] f32 initial Euler state; NULL = drawn by
                                    the library from N(0,1) with noise_seed and a call
                                    counter (not reproducible across handles) */
  const uint8_t* action_mask;    /* [B, H, A] 0/1 applied to the final chunk; NULL = ones */
  float* state_features_out;     /* optional [B, 1, hidden] f32 output; NULL = not written */
} gr00t_inputs;

typedef struct gr00t_head gr00t_head;

/* Create a handle for device `device`: the engine construction of "Single-GPU inference
 * for GR00T-N1.7" (Prepare a request and construct the engine), whose batch capacity is
 * fixed when it is built (max_batch; here also max_vl_len). Checks the config only; no
 * device memory is allocated until gr00t_finalize. Refuses (E_INVALID_ARG) a capacity for
 * which a GEMM operand, a cross block's key/value cache or a workspace buffer would exceed
 * 2^31 - 16 bytes, the range the kernels' 32-bit buffer descriptors address. *out is set
 * to NULL on failure. */
int gr00t_create(const gr00t_config* cfg, int device, gr00t_head** out);

/*
 * Copy one parameter tensor from host memory (the caller may free it on return).
 * `name` is one of the canonical names below, `dtype` is GR00T_F32 (fp32 masters:
 * the library rounds to bf16 with round-to-nearest-even, or quantises DiT matrices
 * to e4m3 with one fp32 scale per output column, scale = max|W[:,o]| / 448) or
 * GR00T_BF16 (raw bf16 bits; not for fp8 matrices). `shape` must equal the
 * canonical shape. Every linear is stored [in, out] (y = x @ W + b), with a leading
 * category axis C for per-embodiment tables:
 *   vlln.gamma [E]  vlln.beta [E]                       (E = vl_dim)
 *   time.w1 [T, D]  time.b1 [D]  time.w2 [D, D]  time.b2 [D]     (T = time_freq_dim)
 *   state_enc.w1 [C, Sd, D]  .b1 [C, D]  .w2 [C, D, D]  .b2 [C, D]
 *   action_enc.w1 [C, A, D] .b1 [C, D] .w2 [C, 2D, D] .b2 [C, D] .w3 [C, D, D] .b3 [C, D]
 *   blocks.{l}.ada.w [D, 2D]  .ada.b [2D]
 *   blocks.{l}.attn.wq [D, D] .bq [D] .wk [Din, D] .bk [D] .wv [Din, D] .bv [D]
 *                  .wo [D, D] .bo [D]      (Din = E for even l, D for odd l)
 *   blocks.{l}.ff.w1 [D, F]  .b1 [F]  .w2 [F, D]  .b2 [D]
 *   out.ada.w [D, 2D]  out.ada.b [2D]  out.proj.w [D, D]  out.proj.b [D]
 *   action_dec.w1 [C, D, D]  .b1 [C, D]  .w2 [C, D, A]  .b2 [C, A]
 * Errors: E_UNKNOWN_WEIGHT, E_SHAPE, E_INVALID_ARG (dtype), E_NOT_FINALIZED (after
 * finalize). Loading a name twice replaces it. Host-only; no device work.
 */
int gr00t_load_weights(gr00t_head* h, const char* name, const void* host_data,
                       gr00t_dtype dtype, const int64_t* shape, int ndim);

/* Check that every weight was loaded (E_MISSING_WEIGHT names the first missing
 * one), upload and pack them, allocate the workspace for (max_batch, max_vl_len)
 * and compute the input-independent per-step tables (timestep embedding, adaLN
 * scale/shift of every block and of the output norm, the timestep half of the
 * action encoder's second linear): the parts of the engine construction ("Single-GPU
 * inference for GR00T-N1.7", Prepare a request and construct the engine) that do not
 * depend on a request; the timestep grid is that of "Model architecture", Inference
 * (denoising). Synchronous. E_OOM if device memory runs out, E_HIP on a runtime failure. */
int gr00t_finalize(gr00t_head* h);

/* Capture the K-step hipGraph for batch B and padded VL length L_pad: the capture
 * profiles of "Single-GPU inference for GR00T-N1.7" (Prepare a request and construct the
 * engine), where every served batch shape must match a captured profile. The graph key is
 * (B, L_pad) alone: the flags are fixed for the handle at create (every graph of a handle
 * is captured with them), and embodiment ids, masks and noise are data read on the device,
 * so one graph serves every id mix and mask pattern (the pages' engine also keys on
 * embodiment categories and mask structures). Needs GR00T_FLAG_USE_GRAPH; synchronous;
 * preparing a shape twice does nothing. */
int gr00t_prepare(gr00t_head* h, int32_t batch, int32_t vl_len);

/*
 * One get_action call: action_pred [B, H, A] f32 (device) = the masked chunk after
 * K Euler steps. Enqueued on `hip_stream` (a hipStream_t; NULL = default stream) and
 * returns without waiting, except in strict mode where the ids are first copied to
 * the host and checked (E_EMBODIMENT). In non-strict mode an out-of-range id is
 * not read: its sample's rows of action_pred are NaN, and a later call on the handle
 * returns E_DEVICE_ERROR once: the first call that finds the copy of the device's
 * count of invalid ids (taken at the end of every call) completed, so the report is not
 * lost when calls are enqueued back to back without synchronising.
 */
int gr00t_get_action(gr00t_head* h, const gr00t_inputs* in, float* action_pred,
                     void* hip_stream);

/*
 * get_action for a call whose vision-language input equals that of the last full
 * get_action (or velocity) call on the handle: System 1 runs at a higher rate than the
 * VLM that feeds it ("GR00T & Embodied AI Models", Dual-system architecture), so several
 * action chunks are drawn from one backbone output. The VL LayerNorm, the key masks and
 * the key/value projection of every cross block are not recomputed: the caches of that
 * call are used as they are. in->vl_features, vl_mask and image_mask are not read (may
 * be NULL); batch and vl_len must equal that call's; state, embodiment_id, noise and
 * action_mask are this call's own. The result equals that of gr00t_get_action with the
 * earlier call's VL inputs. Errors as gr00t_get_action, and E_NO_VL_CACHE when no full
 * call of this (B, L_pad) precedes it (any full call of another shape replaces the cache).
 */
int gr00t_get_action_reuse_vl(gr00t_head* h, const gr00t_inputs* in, float* action_pred,
                              void* hip_stream);

/*
 * Flow-matching training forward and loss of one batch ("GR00T model class", Flow matching
 * diffusion, Training; "Model architecture", Training objective). The draws are inputs:
 * t [B] f32 in [0, 1] (t ~ Beta(1.5, 1) on the pages) and inputs.noise [B, H, A] f32 (N(0, 1)).
 *   x_t    = (1 - t) * noise + t * actions,     v = actions - noise
 *   v_pred = the head's velocity at x_t for each sample's timestep bucket floor(t * buckets)
 *            (the bucket decided in fp32; the timestep embedding, adaLN modulation and the
 *            action encoder's timestep term are computed per sample)
 *   loss   = sum(mask * (v_pred - v)^2) / (sum(mask) + 1e-6), mask = inputs.action_mask
 *            (ones when NULL), summed in double in a fixed order
 * actions [B, H, A] f32, loss [1] f32 and the optional v_pred [B, H, A] f32 are device
 * pointers. Forward only (no gradients). Enqueued on `hip_stream` like gr00t_get_action,
 * not captured in a graph; the first call allocates the per-sample tables
 * (max_batch * ((num_layers + 1) * 2 * hidden + 5 * hidden + time_freq_dim) floats, freed by
 * gr00t_destroy). Errors as gr00t_get_action, E_INVALID_ARG without actions, t or
 * inputs.noise, E_OOM if the tables cannot be allocated. In non-strict mode an invalid id
 * makes the loss NaN.
 */
int gr00t_train_forward(gr00t_head* h, const gr00t_inputs* in, const float* actions, const float* t,
                        float* loss, float* v_pred, void* hip_stream);

/* gr00t_train_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc): the same
 * kernels and results, but the per-sample tables, which gr00t_train_forward allocates on
 * its first call, go to a fixed scratch area of 32 MiB that the library holds on every
 * device it runs on until the process ends. The call allocates nothing (with launch timing
 * off). Limit: batch * ((num_layers + 1) * 2 * hidden + 5 * hidden + time_freq_dim) floats,
 * each of the seven tables rounded up to 256 bytes, at most 32 MiB (76 samples of the
 * 32-block model, hidden 1536); larger batches are refused with GR00T_E_SHAPE before
 * anything is enqueued. Every handle on a device shares that device's area and each call
 * overwrites it (nothing in it needs to start at zero): calls that overlap on one device,
 * on different streams or from different threads, race. Other arguments, semantics and
 * errors as gr00t_train_forward. */
int gr00t_train_forward_noalloc(gr00t_head* h, const gr00t_inputs* in, const float* actions,
                                const float* t, float* loss, float* v_pred, void* hip_stream);

/* Debug and test entry: the velocity v(x = noise, tau_k) of Euler step `step_k`
 * ([B, H, A] f32, device) that get_action adds, times dt = 1/K, to its Euler state at step
 * k ("Model architecture", Inference (denoising): the predicted velocity of the denoising
 * loop), here at x = inputs.noise, without integration or action_mask. With K = 1,
 * get_action = noise + velocity(step 0). inputs.noise must not be NULL. Same stream
 * semantics and errors as gr00t_get_action. */
int gr00t_velocity(gr00t_head* h, const gr00t_inputs* in, int32_t step_k, float* v,
                   void* hip_stream);

/*
 * The per-row e4m3 quantisation of the W8A8 mode (GR00T_FLAG_W8A8), as its GEMMs apply it
 * to their inputs. The pages do not name fp8: the e4m3 weight mode serves the high-batch fp8
 * workload (e4m3 DiT weights with per-output-channel scales), and the format is the OCP
 * 8-bit floating point specification's E4M3 (no infinities, max 448). x: [rows][ld_x] bf16, device, 16-byte aligned; q: [rows][cols] e4m3 codes,
 * device, 8-byte aligned; scale: [rows] f32, device. For each row r:
 * scale[r] = fp32(max_k |x[r][k]|) / 448 (1 for an all-zero row) and q[r][k] = the e4m3
 * code nearest to the fp32 quotient x[r][k] / scale[r] (ties to the even code, magnitudes
 * above 448 saturate, the sign bit follows the quotient's sign), both divisions correctly
 * rounded in fp32. Needs a created handle (for its device and error message); enqueued on
 * `hip_stream`. E_INVALID_ARG for NULL pointers, misaligned x or q, rows < 0, cols not a
 * positive multiple of 8, or ld_x < cols / not a multiple of 8; rows == 0 does nothing.
 */
int gr00t_quantize_e4m3_rows(gr00t_head* h, const void* x, int64_t ld_x, int32_t rows, int32_t cols,
                             uint8_t* q, float* scale, void* hip_stream);

/* Release graphs, device weights and workspace: "Single-GPU inference for GR00T-N1.7",
 * Close the engine (releases the graphs and model references). Waits for the handle's
 * device work to finish first. NULL is a no-op. */
void gr00t_destroy(gr00t_head* h);

/* Message of the last failure on `h` ("" if none); with h == NULL, the last failure
 * of gr00t_create in this thread. The pointer stays valid until the next call on h. */
const char* gr00t_last_error(const gr00t_head* h);

/* Bytes of device memory held by the handle after finalize (weights + workspace). */
size_t gr00t_device_bytes(const gr00t_head* h);

/*
 * Launch timing (tracing support). Kernel launches are bracketed by a pair of HIP
 * events on the call's stream and accumulated per kernel class (vision-language
 * LayerNorm, K/V projection, adaLN, q/qkv projection, self/cross attention, o
 * projection, norm3, MLP up/down, output projection, per-embodiment linears, small
 * kernels, and "steps_graph" for a whole replay of the captured K-step graph).
 *   gr00t_profile_enable: on = 1 times every launch and runs get_action without the
 *     graph; on = 2 keeps the graph, timing the launches outside it and each replay;
 *     on = 0 stops. Enabling clears the totals; E_INVALID_ARG for other values.
 *   gr00t_profile_read: synchronises the recorded events, then returns the number of
 *     launches and their summed duration in ms for class `kclass`; E_INVALID_ARG past
 *     the last class.
 *   gr00t_profile_class_name: static name of class `kclass`, NULL past the last one.
 */
int gr00t_profile_enable(gr00t_head* h, int on);
int gr00t_profile_read(gr00t_head* h, int kclass, int64_t* launches, double* total_ms);
const char* gr00t_profile_class_name(int kclass);

#ifdef __cplusplus
}
#endif
#endif /* GR00T_HEAD_H */

/*
 * vfm.h -- C ABI of the MI355X (gfx950) flow-matching action-expert library.
 *
 * The library runs the denoise loop of a pi0.5-style action expert: N explicit
 * Euler steps of a flow-matching velocity field, each step one pass of a small
 * transformer over the action-chunk tokens that attend to a cached
 * vision+language prefix KV. The PhyAI summary ("Real-Time Physical AI at the
 * Edge, Scalable Rollouts in the Cloud", optimisation and profiling paragraphs)
 * names this ten-step Euler loop of the action expert as the part of pi0.5
 * whose latency is dominated by many small kernel launches; the FlashRT
 * walk-through (component 7, graph capture; the exec/ execution contract)
 * describes the shape of this interface: named device buffers are the only
 * state, the hot path takes device pointers only, and a replay is launched
 * on a stream.
 *
 * Conventions (all entry points):
 *  - Every function returns vfm_status; no C++ exception crosses the ABI.
 *    On failure vfm_last_error() returns a thread-local message.
 *  - Argument, shape, dtype and bound-state checks run on the host before
 *    anything is enqueued, so those errors never touch the device.
 *  - Device pointers are plain HIP device addresses (for instance the
 *    data_ptr() of a torch tensor on a ROCm device); streams are hipStream_t
 *    passed as void* (NULL = the default stream).
 *  - The caller owns every pointer it passes in. Weights are copied and
 *    repacked at create time, so the caller may free its weight tensors after
 *    vfm_expert_create returns. Bound buffers must stay alive until they are
 *    rebound or the expert is destroyed.
 *  - One expert must not be used from two host threads at once.
 *  - Device faults surface as VFM_E_HIP at the call that observes them.
 */
#ifndef VFM_H_
#define VFM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VFM_ABI_VERSION 2

typedef struct vfm_expert vfm_expert;   /* opaque; owned by the library */

typedef enum {
  VFM_OK = 0,
  VFM_E_INVALID_ARG = 1,   /* NULL where a value is required, bad config field, unknown name */
  VFM_E_SHAPE = 2,         /* a shape does not match the config / bound buffers */
  VFM_E_DTYPE = 3,         /* wrong element type for a weight or buffer */
  VFM_E_UNBOUND = 4,       /* denoise needs a buffer that was never bound */
  VFM_E_STATE = 5,         /* call not valid in the expert's current state */
  VFM_E_UNSUPPORTED = 6,   /* valid request this build does not implement */
  VFM_E_OOM = 7,           /* device allocation failed */
  VFM_E_HIP = 8            /* a HIP runtime call or a kernel failed */
} vfm_status;

typedef enum { VFM_F32 = 0, VFM_BF16 = 1, VFM_F16 = 2, VFM_FP8_E4M3 = 3, VFM_I4X2 = 4 } vfm_dtype;

/* Expert variant. VFM_VARIANT_PI05: the time enters every norm (adaptive
 * RMSNorm with gated residuals) and the state embedding is added to every
 * action token. VFM_VARIANT_PI0: one state token (state W_s + b_s) precedes
 * the action tokens and sees only the prefix and itself; the time enters an
 * action-time MLP on [x W_in + b_in ; sincos(t)] (2W -> W -> W, SiLU); the
 * norms are plain RMSNorm with a (1 + w) gain and the residuals ungated. The
 * pages list pi0 and pi0.5 side by side (PhyAI summary, FlashRT forum post)
 * without their equations; both readings are stated with the oracle. pi0 is
 * built for fp32 / bf16 weights, state_dim >= 1, time_emb_dim == width,
 * action_horizon <= 63 and num_layers >= 1. */
typedef enum { VFM_VARIANT_PI05 = 0, VFM_VARIANT_PI0 = 1 } vfm_variant;

/* Storage precision of the per-layer GEMM weights (q/k/v/o/gate/up/down):
 * fp32; bf16; FP8 e4m3 per tensor with FP8 activations (W8A8); int4 with fp16
 * scales per (column, 128-K group) and bf16 activations (W4A16); int8 with
 * fp32 scales per output column and bf16 activations (W8A16); the int4
 * weights of W4A16 with the FP8 activations of W8A8 (W4A8). The PhyAI
 * summary's optimisation paragraph lists these offline quantisation modes.
 * FP8 and W4A8 experts need activation scales (vfm_calibrate or
 * vfm_set_act_scales) before they can denoise. */
typedef enum {
  VFM_W_FP32 = 0, VFM_W_BF16 = 1, VFM_W_FP8 = 2, VFM_W_W4A16 = 3, VFM_W_W8A16 = 4, VFM_W_W4A8 = 5
} vfm_wprec;

typedef struct {
  int32_t abi_version;      /* must equal VFM_ABI_VERSION */
  int32_t num_layers;       /* L >= 0 */
  int32_t width;            /* W, multiple of 256 in [256, 2048] (FP8, W8A16: of 512, W4A16, W4A8: of 1024) */
  int32_t num_q_heads;      /* Hq, multiple of num_kv_heads; Hq * d multiple of 256 (FP8/W8A16 512, W4A16/W4A8 1024) */
  int32_t num_kv_heads;     /* Hkv >= 1 */
  int32_t head_dim;         /* d in {64, 128, 256} (fp32 experts: 64, 128) */
  int32_t mlp_dim;          /* F, multiple of 256 (FP8/W8A16: 512, W4A16/W4A8: 1024), <= 65536 */
  int32_t action_horizon;   /* H, 1..64 action tokens per sample */
  int32_t action_dim;       /* A in {4, 8, 16, 32, 64} */
  int32_t state_dim;        /* S in [0, 4096] (0: no state input) */
  int32_t time_emb_dim;     /* E, even, in [4, 8192] */
  int32_t max_prefix_len;   /* upper bound of P over all binds, 1..4000 */
  int32_t max_batch;        /* upper bound of B over all binds, 1..1024 */
  int32_t num_steps;        /* N in [1, 1000] Euler steps, t from 1 to 0 */
  float rope_base;          /* rotary base, > 0 */
  float rms_eps;            /* RMSNorm epsilon, > 0 */
  int32_t weight_precision; /* vfm_wprec */
  int32_t act_dtype;        /* VFM_F32 (with VFM_W_FP32) or VFM_BF16 (all others) */
  int32_t w4_group_size;    /* 128 for VFM_W_W4A16 and VFM_W_W4A8, ignored otherwise */
  int32_t variant;          /* vfm_variant */
} vfm_config;

/* A named weight handed to vfm_expert_create. Matrices are row-major
 * [in][out] (y = x @ W). dtype is the master type: VFM_F32 when
 * weight_precision is VFM_W_FP32, VFM_BF16 otherwise. */
typedef struct {
  const char* name;
  const void* dev_ptr;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
} vfm_tensor;

/* Returns VFM_ABI_VERSION. */
int vfm_abi_version(void);

/* Thread-local text of the last error on this thread ("" if none). */
const char* vfm_last_error(void);

/* Create an expert from a config and its named weights.
 * pi0.5 names: time_mlp_in.{w,b} [E][W],[W]; time_mlp_out.{w,b} [W][W],[W];
 * in_proj.{w,b} [A][W],[W]; state_proj.{w,b} [S][W],[W] (S > 0 only);
 * layers.{l}.attn_norm.mod.{w,b} and layers.{l}.mlp_norm.mod.{w,b} [W][3W],[3W]
 * (columns [scale | shift | gate]); layers.{l}.{q,k,v}.w [W][H*d] (head-major
 * columns); layers.{l}.o.w [Hq*d][W]; layers.{l}.{gate,up}.w [W][F];
 * layers.{l}.down.w [F][W]; final_norm.mod.{w,b}; out_proj.{w,b} [W][A],[A].
 * pi0 names: time_mlp_in.{w,b} [2W][W],[W] (rows 0..W-1 take the action
 * embedding, rows W..2W-1 the time embedding); time_mlp_out.{w,b};
 * in_proj.{w,b}; state_proj.{w,b}; layers.{l}.attn_norm.w and
 * layers.{l}.mlp_norm.w [W] (the w of a (1 + w) gain); the same q/k/v/o/
 * gate/up/down; final_norm.w [W]; out_proj.{w,b}.
 * Synchronous on `stream`: copies, repacks and (for FP8 / W4A16) quantises the
 * weights on the device and precomputes the time-conditioning table for the
 * N fixed times t_k = (N-k)/N. All workspace for max_batch / max_prefix_len
 * is allocated here; denoise never allocates. The workspace is dominated by
 * a write-once activation ring of N L slabs, each slab (4 KiB-aligned parts)
 * Mp W (2 a) + B Hq d 64 a + 2 B Hkv d 64 a + Mp Hq d a + Mp F a bytes (plus
 * Mp W a for pi0), with Mp = round_up(max_batch T, 64), T the suffix tokens
 * per sample, a the activation bytes (2 bf16, 4 f32); about 225 MB for the
 * pi0.5 expert at batch 1. A configuration whose workspace would exceed
 * 64 GiB fails with VFM_E_UNSUPPORTED before anything is allocated.
 * Errors: VFM_E_INVALID_ARG (config field out of range, missing or unknown
 * name), VFM_E_SHAPE, VFM_E_DTYPE, VFM_E_UNSUPPORTED (a buffer beyond 2 GiB,
 * or the workspace beyond 64 GiB), VFM_E_OOM, VFM_E_HIP. On error *out is NULL. */
vfm_status vfm_expert_create(const vfm_config* cfg, const vfm_tensor* weights, int32_t n_weights,
                             void* stream, vfm_expert** out);

/* Bind a named device buffer. Names and layouts:
 *   "prefix_k", "prefix_v": [L][B][P][Hkv][d], act_dtype, the cached prefix
 *      keys (already position-encoded) and values of every layer;
 *   "noise":   [B][H][A] f32, the sample at t = 1;
 *   "state":   [B][S] f32 (S > 0 only);
 *   "actions": [B][H][A] f32, receives the sample at t = 0.
 * B (1..max_batch) and P (1..max_prefix_len) are taken from the prefix_k
 * shape; every other buffer must agree. Pointers must be 16-byte aligned.
 * Host-only validation; nothing is enqueued. Errors: VFM_E_INVALID_ARG,
 * VFM_E_SHAPE, VFM_E_DTYPE. */
vfm_status vfm_bind(vfm_expert* ex, const char* name, void* dev_ptr, int32_t dtype, int32_t ndim,
                    const int64_t* shape);

/* Run the N-step denoise loop on `stream` (asynchronous). noise / state /
 * actions may be NULL to use the bound buffers; non-NULL pointers replace
 * the bound ones for this call and must have the bound shapes. actions may
 * alias noise. Errors: VFM_E_UNBOUND (prefix or a needed buffer not bound),
 * VFM_E_STATE, VFM_E_HIP (launch failure or a fault seen from an earlier
 * call). */
vfm_status vfm_denoise(vfm_expert* ex, const float* noise, const float* state, float* actions,
                       void* stream);

/* Options (string key/value), host-only:
 *   "launch_mode": "auto" (default), "persistent", "graph" or "eager".
 *       "persistent": one cooperative launch per denoise with device-wide
 *       phase barriers; "graph": one kernel per phase, captured into a
 *       hipGraph per shape and pointer set and replayed; "eager": the same
 *       kernels launched directly. With bf16 weights and B x T >= 256 rows
 *       the graph and eager modes run large-batch kernels (128-column GEMM
 *       tiles, 256-column tiles for gate/up, single-pass attention). "auto"
 *       chooses, per call, graph launch where those apply and the persistent
 *       kernel otherwise.
 *   "large_m_tiles": "auto" (default), "narrow" or "wide": the large-batch
 *       GEMM tiles of the graph and eager modes: 256 columns x 224 or 256
 *       tokens (one workgroup per compute unit, a direct-to-LDS operand
 *       ring) for gate/up only, for no GEMM, or for every GEMM whose column
 *       count is a multiple of 256. Results agree to rounding (K splits
 *       differ). Invalidates captured graphs.
 *   "persistent_launch": "cooperative" (default) or "plain": how the
 *       persistent kernel is launched. "plain" is an ordinary launch of the
 *       same grid (one workgroup per compute unit, from the occupancy query);
 *       it relies on the device being otherwise idle so that every
 *       workgroup is resident. If one is not, the device-wide barrier gives
 *       up after a bounded spin and the next vfm_check / vfm_denoise
 *       reports VFM_E_HIP. Used where a tool cannot follow cooperative
 *       launches (kernel profilers).
 *   "fused_norms": "auto" (default), "1" or "0": the persistent
 *       kernel of a pi0.5 expert with bf16, W4A16 or W8A16 weights (width a
 *       multiple of 256, at most 1024; the shift W table is built from the
 *       weights the GEMMs multiply by)
 *       folds the adaptive RMSNorms into the GEMMs next to them (the
 *       residual + norm fusion of the FlashRT walk-through, component 8):
 *       the o and down projections finish the gated residual in the
 *       epilogue of the last K split of each column group to arrive and
 *       write y = h (1 + scale) of the next norm with per-16-column sums of
 *       squares; qkv and gate/up apply r = 1 / sqrt(mean(h^2) + eps) and a
 *       create-time shift W table. The same kernel merges the attention key
 *       splits inside the attention phase (per-head arrival counters) and
 *       starts each attention unit once its head's qkv tiles are stored
 *       (per-head tile counters): four device-wide barriers per layer
 *       instead of eight. Results agree with "0" to bf16 rounding of the
 *       GEMM inputs. "auto" folds for calls of at most 128 rows (batch
 *       times rows per sample: pi0.5 batch 1 and 2), where the barriers
 *       dominate; larger calls are faster with separate norm phases (the
 *       split-sum exchanges and per-row scaling outweigh the barriers
 *       saved), which "1" overrides. VFM_E_UNSUPPORTED for "1" on other
 *       experts ("auto" then keeps separate norm phases).
 *   "attn_merge": "1" (default) or "0": every persistent kernel merges
 *       the attention key splits inside the attention phase (per-head
 *       arrival counters, one 128-byte line each) and starts each attention
 *       unit once its head's qkv tiles are stored (per-head tile counters),
 *       so the barriers after qkv and after attention go; "0" runs a combine
 *       phase between device-wide barriers instead (and, since the
 *       folded-norm kernel needs the in-place merge, separate norm phases).
 *       Results are bitwise the same with separate norm phases.
 *   "xcd_local": "1" (default) or "0": with folded norms, the K-split
 *       units of one o / down column group all run on one XCD (unit index
 *       mod 8, checked at kernel start from the hardware XCD id; a launch
 *       whose workgroups are placed otherwise uses the device-wide path),
 *       and exchange their partial sums through that XCD's L2 instead of
 *       the device coherence point; likewise the key splits of attention
 *       head j and the merge of its rows run on XCD j mod 8. "splits"
 *       (diagnostics) keeps only the o / down part. Results are bitwise
 *       the same for every value.
 *   "trace": "1" / "0": record a timeline of the persistent kernel's phase
 *       barriers (workgroup 0), read with vfm_export("trace").
 *   "graph_cache": "1" .. "64" (default 8): graph mode keeps one captured
 *       graph per key (B, P and the noise / state / actions / prefix
 *       pointers), at most this many, dropping the least recently used (the
 *       FlashRT walk-through's Graph object: an exact-key variant table with
 *       LRU). Alternating between a few buffer sets then replays without
 *       capturing again.
 * Errors: VFM_E_INVALID_ARG for an unknown key or value. */
vfm_status vfm_set_option(vfm_expert* ex, const char* key, const char* value);

/* FP8 and W4A8 experts: one measurement pass, as in the FlashRT walk-through
 * (component 6, calibration): run the whole denoise loop once on the bound
 * buffers (prefix_k, prefix_v, noise, state; `actions` is overwritten) in
 * bf16, with the dequantised weights materialised in bf16 for the pass
 * only, record the largest |input| of every GEMM (4 per layer, over all
 * steps), and set act_scale = amax / 448 (1 where amax is 0); the GEMM
 * epilogues then use alpha = act_scale * weight_scale (W4A8: act_scale, the
 * group scales being applied inside the GEMM). Such an expert's denoise
 * returns VFM_E_STATE until this or vfm_set_act_scales has run.
 * Synchronous on `stream`; invalidates captured graphs.
 * Errors: VFM_E_STATE (not FP8 / W4A8), VFM_E_UNBOUND / VFM_E_SHAPE
 * (buffers), VFM_E_OOM, VFM_E_HIP. */
vfm_status vfm_calibrate(vfm_expert* ex, void* stream);

/* Set the n = 4 * L FP8 activation scales directly (host array, order per
 * layer: qkv input, o input, gate/up input, down input; each > 0), e.g.
 * scales cached from an earlier calibration. Synchronises the device.
 * Errors: VFM_E_STATE (not FP8 / W4A8), VFM_E_SHAPE (n != 4 * L),
 * VFM_E_INVALID_ARG (a scale not positive and finite). */
vfm_status vfm_set_act_scales(vfm_expert* ex, const float* scales, int32_t n);

/* Copy a tensor the library holds, as float32, to host memory `dst`
 * (`bytes` must equal 4 * element count):
 *   a per-layer GEMM weight by its create-time name (e.g. "layers.3.q.w"):
 *      the value the kernels multiply by, i.e. dequantised for the quantised formats,
 *      row-major [in][out];
 *   "mod_table": [N][2L+1][3][W], (scale, shift, gate) of every norm at
 *      every step (norm order attn_0, mlp_0, ..., final);
 *   "weight_scales" (FP8), "act_scales" (FP8, W4A8): [L][4] per-GEMM scales
 *      (qkv, o, gate/up, down); act_scales needs a calibration first;
 *   "trace": the phase timeline of the last persistent call (option "trace");
 *   "persistent_plan": 6 int32 (not float32): whether the persistent kernel
 *      runs with folded norms (0 / 1), its device-wide barriers per call,
 *      the K splits of the o and down projections, whether their split
 *      sums are exchanged through one XCD's L2 (0 / 1; option "xcd_local"),
 *      and whether the attention splits are merged in place (0 / 1; option
 *      "attn_merge"),
 *      at the bound batch and prefix; VFM_E_UNBOUND without prefix_k,
 *      VFM_E_STATE when the expert would not run the persistent kernel there.
 * Synchronous. Errors: VFM_E_INVALID_ARG (unknown name), VFM_E_SHAPE,
 * VFM_E_STATE. */
vfm_status vfm_export(vfm_expert* ex, const char* name, void* dst, size_t bytes);

/* Measurement helper (not part of the denoise path): copy `bytes` (a multiple
 * of 16 below 2 GiB) from `src` to `dst` (device, 16-byte aligned, not
 * overlapping) with loads of cache policy `policy`: 0 plain, 1 sc0
 * (workgroup scope), 16 sc1 (device scope); stores plain. A kernel of known
 * traffic against which HBM counters are scaled for each load policy the
 * kernels use. Asynchronous on `stream`. Errors: VFM_E_INVALID_ARG, VFM_E_HIP. */
vfm_status vfm_copy_probe(const void* src, void* dst, size_t bytes, int32_t policy, void* stream);

/* Wait for `stream` and report any device-side failure of earlier denoise
 * calls (a launch error, or a phase barrier that timed out and stopped the
 * persistent kernel early): VFM_E_HIP with a message. */
vfm_status vfm_check(vfm_expert* ex, void* stream);

/* Synchronise the expert's work and free everything it owns. NULL-safe. */
vfm_status vfm_expert_destroy(vfm_expert* ex);

/* Diagnostics of the streaming batch-1 kernel (launch_mode "stream"): copy
 * the raw bytes of one of its internal buffers to host memory `dst`
 * (synchronous; `bytes` must equal the buffer size). Names: "slab" (the
 * intermediates of step k, layer l at index = k L + l: y_attn, norm sums of
 * squares, q, k, transposed v, attention output, y_mlp, sums, MLP
 * activation), "h" (residual stream, [64][W] f32), "s_emb", "vt" (prefix
 * values transposed), "apart" / "aml" (attention split outputs and their
 * (max, sum)), "shw_q" / "shw_g" (create-time shift x W tables);
 * "slab_layout" writes 10 uint64: the byte offsets of the nine slab
 * sections in that order, then the slab size. For tests; not a hot-path call.
 * Errors: VFM_E_INVALID_ARG, VFM_E_STATE (no streaming state), VFM_E_SHAPE,
 * VFM_E_HIP. */
vfm_status vfm_stream_debug(vfm_expert* ex, const char* name, int32_t index, void* dst, size_t bytes);

/* Execution-state capsules. The FlashRT-PAI introduction (its third
 * mechanism, execution-state capsules) and the FlashRT walk-through (serving
 * hosts: graph-replay-native capsules with snapshot, restore, fork and time
 * travel) describe fast snapshots of a pipeline's persistent state. Here that
 * state is the contents of the bound buffers (prefix_k, prefix_v, noise,
 * state, actions: whichever are bound when the capsule is created) plus, for
 * FP8 experts, the activation scales. Taking and putting back a snapshot is
 * a handful of stream-ordered device-to-device copies: no allocation, no
 * host synchronisation, no graph invalidation (the bound pointers do not
 * change). Keep several capsules for time travel; restore one into another
 * expert of the same layout to fork a rollout. */
typedef struct vfm_capsule vfm_capsule;   /* opaque; owned by the caller via create/destroy */

/* Allocate a capsule for the expert's current bindings: one device buffer
 * per bound buffer, of the same size. prefix_k must be bound (it fixes B and
 * P). The capsule holds no state until vfm_capsule_save. Allocates (not for
 * use inside a tight loop); nothing is enqueued.
 * Errors: VFM_E_INVALID_ARG (NULL), VFM_E_UNBOUND, VFM_E_OOM. On error *out
 * is NULL. */
vfm_status vfm_capsule_create(vfm_expert* ex, vfm_capsule** out);

/* Snapshot: enqueue on `stream` copies of every buffer in the capsule from
 * the expert's bound buffer into the capsule (asynchronous; ordered after
 * earlier work on `stream`, e.g. a denoise that writes `actions`), and
 * record the FP8 activation scales. The expert must have the layout the
 * capsule was made for: same L, Hkv, d, H, A, S and activation type, same B
 * and P, and every buffer of the capsule bound with the same size.
 * Errors: VFM_E_INVALID_ARG, VFM_E_UNBOUND, VFM_E_SHAPE (layout differs),
 * VFM_E_STATE (FP8 capsule with a non-FP8 expert or the reverse), VFM_E_HIP. */
vfm_status vfm_capsule_save(vfm_expert* ex, vfm_capsule* cap, void* stream);

/* Restore / fork: enqueue on `stream` copies from the capsule into the bound
 * buffers of `ex`, which may be the expert the capsule was saved from or
 * another one of the same layout (a fork; its weights may differ). When
 * both are FP8 experts, the expert's activation scales are set to the
 * capsule's first (synchronous, only if they differ). The capsule is not
 * changed and can be restored any number of times.
 * Errors: VFM_E_INVALID_ARG, VFM_E_STATE (never saved), VFM_E_UNBOUND,
 * VFM_E_SHAPE, VFM_E_HIP. */
vfm_status vfm_capsule_restore(vfm_expert* ex, const vfm_capsule* cap, void* stream);

/* Device bytes the capsule holds. Errors: VFM_E_INVALID_ARG. */
vfm_status vfm_capsule_bytes(const vfm_capsule* cap, size_t* bytes);

/* Synchronise the device and free the capsule. NULL-safe. */
vfm_status vfm_capsule_destroy(vfm_capsule* cap);

/* ------------------------------------------------------------------------
 * Prefix producer. The pages treat the vision + language prefix as the part
 * of pi0 / pi0.5 that runs once per observation before the action expert,
 * which reads it only through the cached per-layer keys and values (PhyAI
 * summary, profiling paragraph: the expert's share of batch-1 latency is what
 * remains after this pass; the FlashRT forum post lists Pi0 / Pi0.5 as its
 * flagship VLA integrations). This is that pass for a Gemma-shaped decoder:
 * per layer, x -> RMSNorm with a (1 + w) gain -> fused Q/K/V projection with
 * rotary encoding (half-split pairs, positions 0..P-1) -> bidirectional
 * grouped-query attention over the sample's P tokens -> o projection ->
 * residual -> RMSNorm (1 + w) -> GeGLU (tanh GELU) MLP -> residual. Its
 * outputs are every layer's rotary-encoded keys and values, written straight
 * into the buffers the expert binds as "prefix_k" / "prefix_v". The last
 * layer's attention output and MLP reach no output and are not computed.
 * ------------------------------------------------------------------------ */
typedef struct vfm_prefix vfm_prefix;   /* opaque; owned by the library */

typedef struct {
  int32_t abi_version;      /* must equal VFM_ABI_VERSION */
  int32_t num_layers;       /* L in [1, 256]; the expert that reads the K/V has the same L */
  int32_t width;            /* W, multiple of 128 in [128, 4096] */
  int32_t num_q_heads;      /* Hq, multiple of num_kv_heads, <= 64; Hq * d multiple of 128 */
  int32_t num_kv_heads;     /* Hkv >= 1 */
  int32_t head_dim;         /* d in {64, 128, 256} */
  int32_t mlp_dim;          /* F, multiple of 64 in [64, 65536] */
  int32_t max_prefix_len;   /* upper bound of P over all runs, 1..8192 */
  int32_t max_batch;        /* upper bound of B over all runs, 1..256 */
  float rope_base;          /* rotary base, > 0 */
  float rms_eps;            /* RMSNorm epsilon, > 0 */
} vfm_prefix_config;

/* Create a prefix producer from bf16 weights (row-major [in][out]):
 * layers.{l}.attn_norm.w [W], layers.{l}.{q,k,v}.w [W][H*d] (head-major
 * columns), layers.{l}.o.w [Hq*d][W], layers.{l}.mlp_norm.w [W],
 * layers.{l}.{gate,up}.w [W][F], layers.{l}.down.w [F][W]; norm weights are
 * the w of the (1 + w) gain. Every name is required (also the last layer's,
 * though only its attn_norm, k and v are used). Synchronous on `stream`:
 * repacks the weights into MFMA operand order and allocates all workspace for
 * max_batch x max_prefix_len tokens; run never allocates. The caller may free
 * its weight tensors afterwards.
 * Errors: VFM_E_INVALID_ARG (config, missing / unknown / NULL weight),
 * VFM_E_SHAPE, VFM_E_DTYPE (weights not bf16), VFM_E_UNSUPPORTED (a buffer
 * beyond 2 GiB), VFM_E_OOM, VFM_E_HIP. On error *out is NULL. */
vfm_status vfm_prefix_create(const vfm_prefix_config* cfg, const vfm_tensor* weights, int32_t n_weights,
                             void* stream, vfm_prefix** out);

/* Run the pass on `stream` (asynchronous): embeds [B][P][W] bf16 token
 * embeddings (device), prefix_k / prefix_v [L][B][P][Hkv][d] bf16 outputs
 * (device; the expert's "prefix_k" / "prefix_v" layout). Pointers 16-byte
 * aligned; the outputs must not alias the input. Errors: VFM_E_INVALID_ARG
 * (NULL or misaligned pointer), VFM_E_SHAPE (B or P outside [1, max]),
 * VFM_E_HIP (launch failure). */
vfm_status vfm_prefix_run(vfm_prefix* pre, const void* embeds, int32_t batch, int32_t prefix_len,
                          void* prefix_k, void* prefix_v, void* stream);

/* vfm_prefix_run for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same pass with the same arguments and results, but its workspace
 * (residual stream, K-split partial sums, normalised and attention operands,
 * activations, queries, transposed values, rotary table) lives in one static
 * 64 MiB device array per GPU instead of the producer's buffers. It calls no
 * hipMalloc, hipFree or allocating library routine; the array's address is
 * looked up once per device on the first call there. Workspace needed:
 * round_up(B P, 128) x (W (6 + 4 S) + 4 Hq d + 2 F) bytes (S the K splits,
 * at most 8) + B Hkv d round_up(P, 32) x 2 + P d x 4 bytes, each piece
 * rounded up to 256; more than 64 MiB fails with VFM_E_UNSUPPORTED before
 * any launch. Every call on a GPU shares that GPU's array and clears what
 * must start at zero itself; calls that overlap on one GPU (different
 * streams, different producers) race and must be ordered by the caller.
 * Errors: those of vfm_prefix_run, VFM_E_UNSUPPORTED, VFM_E_HIP (symbol
 * lookup or launch failure). */
vfm_status vfm_prefix_run_noalloc(vfm_prefix* pre, const void* embeds, int32_t batch, int32_t prefix_len,
                                  void* prefix_k, void* prefix_v, void* stream);

/* Options (string key/value), host-only:
 *   "gate_up_tiles": "wide" (default) or "narrow": the gate/up GEMM on
 *       256-column tiles (one workgroup per compute unit, a direct-to-LDS
 *       operand ring; used where N is a multiple of 256 and K of 64) or on
 *       the 128 x 128 tiles of the other GEMMs. Results agree to rounding.
 *   "down_tiles": "wide" (default) or "narrow": the down projection on the
 *       same 256-column tiles with K splits (up to 8, partial sums added by
 *       the next norm) where one round of tiles fills at least 192 compute
 *       units, every split has at least 1024 K and the tiles cover the
 *       padded token rows, or on the 128 x 128 tiles. Results agree to
 *       rounding (a different summation order).
 *   "o_tiles": "auto" (default) or "full": the o projection on 128-token x
 *       64-column tiles with half the K splits where 128 x 128 tiles would
 *       split K, or on 128 x 128 tiles. Results agree to rounding.
 *   "qkv_tiles": "auto" (default) or "full": the fused QKV projection on
 *       128-token x 64-column tiles where 128 x 128 tiles would number at
 *       most 128 (half the compute units), or always on 128 x 128 tiles.
 *       Results are the same (each output's sum is formed the same way).
 * Errors: VFM_E_INVALID_ARG for a NULL argument or an unknown key or value. */
vfm_status vfm_prefix_set_option(vfm_prefix* pre, const char* key, const char* value);

/* Synchronise the device and free everything the producer owns. NULL-safe. */
vfm_status vfm_prefix_destroy(vfm_prefix* pre);

/* ------------------------------------------------------------------------
 * Plan. The FlashRT walk-through (its exec/ C ABI: Buffer, Graph, Plan)
 * describes a Plan as a DAG of graphs across streams that carries data
 * dependencies only, with no priorities or preemption, and the FlashRT-PAI
 * introduction's execution contract adds per-stage update rates, reuse of
 * state across decisions and selective refresh. Here a plan is a list of
 * stages, each the prefix pass of a producer, the denoise call of an expert
 * or an adopted graph, each with an update rate: stage i runs at tick t when
 * t >= offset_i and (t - offset_i) is a multiple of every_i, so a prefix stage
 * with every = 5 refreshes the prefix K/V on every fifth control tick and the
 * expert stages in between reuse it. Dependencies are derived, not declared:
 * every stage has the device byte ranges it reads and writes (the producer's
 * embeddings and K/V outputs; the expert's bound prefix_k / prefix_v / noise /
 * state / actions, or the pointers given at add time; an adopted graph's
 * declared ranges) and the private workspace of its producer or expert. Within
 * a tick, a due stage waits for every earlier due stage (in add order) whose
 * writes overlap its reads or writes, or whose reads overlap its writes, or that
 * uses the same producer or expert, or that vfm_plan_add_edge names; other
 * stages run concurrently on their own streams. An expert in persistent
 * launch mode holds every compute unit with device-wide barriers, so it also
 * waits for every earlier due stage, and every later one waits for it. Each
 * tick is ordered after earlier work on the caller's stream and before later
 * work on it (the tick forks from and joins back into that stream), so ticks
 * do not overlap one another.
 * Thread safety: a plan, and the producers and experts in it, must not be used
 * from two threads at once.
 * ------------------------------------------------------------------------ */
typedef struct vfm_plan vfm_plan;   /* opaque; owned by the caller via create/destroy */

typedef struct {
  const void* ptr;   /* device address */
  size_t bytes;
} vfm_range;

/* Create an empty plan. Host only (streams and events are made at the first
 * run). Errors: VFM_E_INVALID_ARG (out is NULL). */
vfm_status vfm_plan_create(vfm_plan** out);

/* Add a stage that runs vfm_prefix_run(pre, embeds, batch, prefix_len,
 * prefix_k, prefix_v) at its ticks. Reads embeds ([B][P][W] bf16), writes
 * prefix_k and prefix_v ([L][B][P][Hkv][d] bf16 each). every >= 1,
 * 0 <= offset < every. *stage receives the stage index (0, 1, ... in add
 * order). The producer must outlive the plan.
 * Errors: VFM_E_INVALID_ARG (NULL, misaligned pointer, bad rate),
 * VFM_E_SHAPE (batch or prefix_len outside the producer's limits). */
vfm_status vfm_plan_add_prefix(vfm_plan* pl, vfm_prefix* pre, const void* embeds, int32_t batch, int32_t prefix_len,
                               void* prefix_k, void* prefix_v, int32_t every, int32_t offset, int32_t* stage);

/* Add a stage that runs vfm_denoise(ex, noise, state, actions) at its ticks.
 * NULL pointers mean the expert's bound buffers as bound when the tick runs
 * (rebinding between ticks is seen). Reads prefix_k, prefix_v, noise and
 * state; writes actions. The expert must outlive the plan.
 * Errors: VFM_E_INVALID_ARG (NULL expert, misaligned pointer, bad rate). */
vfm_status vfm_plan_add_denoise(vfm_plan* pl, vfm_expert* ex, const float* noise, const float* state, float* actions,
                                int32_t every, int32_t offset, int32_t* stage);

/* Adopt a graph captured elsewhere (a hipGraphExec_t instantiated on this
 * device, e.g. a camera pre-processing step or a torch-captured graph): the
 * stage launches it with hipGraphLaunch at its ticks. reads / writes list
 * the device ranges the graph reads and writes (n may be 0). The graph
 * stays owned by the caller and must outlive the plan.
 * Errors: VFM_E_INVALID_ARG (NULL graph, NULL range list with n > 0, a range
 * with a NULL pointer or 0 bytes, bad rate). */
vfm_status vfm_plan_add_graph(vfm_plan* pl, void* graph_exec, const vfm_range* reads, int32_t n_reads,
                              const vfm_range* writes, int32_t n_writes, int32_t every, int32_t offset,
                              int32_t* stage);

/* Declare that stage `to` depends on stage `from` through memory the plan
 * cannot see (from < to). Applies at ticks where both run.
 * Errors: VFM_E_INVALID_ARG (index out of range, from >= to). */
vfm_status vfm_plan_add_edge(vfm_plan* pl, int32_t from, int32_t to);

/* Host-only query: the stages that stage `stage` waits for at tick `tick`
 * (ascending), written to deps[0 .. min(*n, cap) - 1]; *n = their count, and
 * -1 if the stage does not run at that tick. Errors: VFM_E_INVALID_ARG,
 * VFM_E_UNBOUND (an expert stage whose buffers are not bound). */
vfm_status vfm_plan_deps(vfm_plan* pl, int64_t tick, int32_t stage, int32_t* deps, int32_t cap, int32_t* n);

/* Run tick `tick` (>= 0): enqueue every due stage, in add order, each on its
 * own stream after the stages it depends on; `stream` then waits for all of
 * them. Asynchronous; no allocation after the first run (graph-mode experts
 * capture their graph on first use of a shape and pointer set). If a stage
 * fails to enqueue, the stages already enqueued are still joined into
 * `stream` and the stage's error is returned. Errors: VFM_E_INVALID_ARG,
 * any error of the stages' own calls. */
vfm_status vfm_plan_run(vfm_plan* pl, int64_t tick, void* stream);

/* Synchronise the plan's streams and free them. NULL-safe. */
vfm_status vfm_plan_destroy(vfm_plan* pl);

#ifdef __cplusplus
}
#endif

#endif /* VFM_H_ */

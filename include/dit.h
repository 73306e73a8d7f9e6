/*
 * dit.h -- C ABI of the MI355X (gfx950) diffusion-transformer block forward.
 *
 * The library computes the non-causal DiT block that a diffusion denoise loop
 * runs at every step: AdaLN shift/scale/gate modulation around RMSNorm or
 * LayerNorm, a fused QKV GEMM, NeoX rotate_half RoPE from a per-row cos/sin
 * cache, packed varlen non-causal attention over cu_seqlens, the output
 * projection, a gated residual, a gated-SiLU MLP and a second gated residual
 * (page "port the MiniMax-H3 omni-modal video+audio DiT", section "The
 * device-resident forward (W2b)"; page "the 2.4B fp32 DiT onto the device,
 * staged once", section "What moved, and onto what").
 *
 * Conventions for every call:
 *   - Every function returns a dit_status.  Nothing aborts the process and no
 *     C++ exception crosses this boundary; dit_last_error() gives a message
 *     naming the offending argument or tensor (thread-local).
 *   - "dev" pointers are HIP device pointers on the current device; "host"
 *     pointers are ordinary host memory.  The library allocates no device
 *     memory: weights live in a caller-allocated slab, batch tables in a
 *     caller-allocated buffer, scratch in a caller-allocated workspace.
 *   - Device work is enqueued on the hipStream_t passed in (NULL = the default
 *     stream) and is asynchronous; no forward call synchronises the host.
 *     Host buffers passed to staging calls are copied before those calls return.
 *   - Matrices are row-major.  Weights use the nn.Linear layout [out, in].
 *   - A sticky HIP error (for example an illegal address) is reported as
 *     DIT_E_HIP; the device context is then unusable and there is no recovery.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dit_stream_t; /* same type as hipStream_t */

typedef enum dit_status {
  DIT_OK = 0,
  DIT_E_INVALID = 1,        /* a bad argument; the message names it */
  DIT_E_STATE = 2,          /* call out of order (stage after finalize, forward before finalize) */
  DIT_E_UNKNOWN_WEIGHT = 3, /* staging a name outside the weight contract */
  DIT_E_SHAPE = 4,          /* a weight's shape differs from the contract */
  DIT_E_DTYPE = 5,          /* a weight's dtype cannot be staged into its slot */
  DIT_E_MISSING_WEIGHT = 6, /* finalize found a tensor never staged; the message names it */
  DIT_E_WORKSPACE = 7,      /* a caller buffer is smaller than the required size */
  DIT_E_HIP = 8,            /* a HIP runtime error */
  DIT_E_UNSUPPORTED = 9     /* a shape outside what the kernels handle (message says which) */
} dit_status;

enum { DIT_F32 = 0, DIT_BF16 = 1, DIT_F64 = 2 /* residual stream of an fp32 model only */,
       DIT_MXFP8 = 3 /* OCP E4M3 values with one E8M0 scale per 32 along K (dit_gemm, dit_quantize_mx8) */,
       DIT_MXFP4 = 4 /* OCP E2M1 values, two per byte (even K in the low nibble), one E8M0 scale per 32
                        along K (dit_gemm's weight operand, dit_quantize_mx4) */ };
/* Format of the four block GEMMs of a bf16-stream model: the stream dtype;
 * MXFP8 re-quantized operands (weights at staging, activations before each
 * GEMM) on the scaled fp8 matrix cores; or MXFP4 weights (re-quantized at
 * staging) against the same MXFP8 activations on the same matrix cores
 * (page "port the MiniMax-H3 omni-modal video+audio DiT", update "NVFP4 arm
 * grounded": 4-bit weights with block scales; here W4A8, the FP4 operand
 * needing an MX partner). */
enum { DIT_GEMM_STREAM = 0, DIT_GEMM_MXFP8 = 1, DIT_GEMM_MXFP4 = 2 };
enum { DIT_NORM_RMS = 0, DIT_NORM_LAYER = 1 };
enum { DIT_MLP_GATE_UP = 0, DIT_MLP_VALUE_GATE = 1 };
enum { DIT_IO_NONE = 0, DIT_IO_PATCH3D = 1, DIT_IO_CHANNEL_MAJOR = 2 };
/* Row layout of the fused qkv projection: [q_all | k_all | v_all] (the DiT's),
 * or per head [q | k | v of head 0 | q | k | v of head 1 | ...] (the video VAE
 * decoder's ViT; page "port the MiniMax-H3 omni-modal video+audio DiT", update
 * "video-VAE decoder block ported": same size, a wrong reading raises no
 * error).  A per-head weight is reordered at stage time. */
enum { DIT_QKV_CONCAT = 0, DIT_QKV_PER_HEAD = 1 };
/* Position grid of a modality's rotary angles: integer positions from 0, or
 * per axis the centre of cell i of [-1, 1) split in n, (2i + 1)/n - 1, scaled
 * by 2 pi (the ViT decoder's ND rotary embedding; same page, update "video-VAE
 * ViT3D decoder complete"). */
enum { DIT_ROPE_INTEGER = 0, DIT_ROPE_CENTERED = 1 };

#define DIT_MAX_MODALITIES 4
#define DIT_MAX_SEGMENTS 64
#define DIT_MAX_COND 64

/* One modality: its in/out projection geometry and its rope axes. */
typedef struct dit_modality {
  int io;          /* DIT_IO_*; must be DIT_IO_NONE iff dit_config.io == 0 */
  int channels;    /* latent channels C */
  int patch[3];    /* (pt, ph, pw) for DIT_IO_PATCH3D, else (1,1,1) */
  int n_axes;      /* 1 or 3 position axes */
  int axis_dim[3]; /* rotary sub-dimension per axis; sums to rot_dim; each even */
  int rope_grid;   /* DIT_ROPE_* */
} dit_modality;

/* Model shape.  All fields are read at dit_model_create and copied. */
typedef struct dit_config {
  int n_blocks, hidden, n_heads, head_dim, ffn;
  int norm;          /* DIT_NORM_*: row norm without affine weights */
  float norm_eps;
  int mlp;           /* DIT_MLP_GATE_UP: mlp.in rows are [gate | up];
                        DIT_MLP_VALUE_GATE: [value | gate], swapped at stage time */
  int rot_dim;       /* rotary dims at the start of each head (<= head_dim, even) */
  double theta;      /* rope base */
  int stream_dtype;  /* DIT_F32 or DIT_BF16: dtype of block weights and of the GEMM operands */
  int cond_dim;      /* width d_t of the conditioning vector feeding the AdaLN linears */
  int n_mod;         /* modalities (one AdaLN linear and one projection pair each) */
  int io;            /* 1: latents in / velocities out through fp32 projections; 0: tokens in/out */
  dit_modality mod[DIT_MAX_MODALITIES];
  int gemm_format;   /* DIT_GEMM_*: DIT_GEMM_MXFP8 / _MXFP4 need a bf16 stream and hidden, ffn multiples of 128
                        (the low-precision arm; page "port the MiniMax-H3 omni-modal video+audio DiT",
                        update "NVFP4 arm grounded": the pages' is NVFP4, this GPU's matrix cores take MX) */
  int qkv_layout;    /* DIT_QKV_* */
  int qk_norm;       /* 1: q and k RMS-normalised over each head (eps norm_eps, no weight) before RoPE,
                        as the ViT decoder block (same page, update "video-VAE decoder block ported");
                        fp32 stream only */
} dit_config;

/* One document of a packed batch: a contiguous run of tokens of one modality
 * with one position grid and one modulation row.  Tokens are counted by the
 * grid: grid[0] (1 axis) or grid[0]*grid[1]*grid[2] (3 axes, raster order with
 * the last axis fastest).  Segments are packed end to end in array order. */
typedef struct dit_segment {
  int modality;  /* index into dit_config.mod */
  int cond_row;  /* modulation row of every token in the segment */
  int grid[3];   /* token grid; unused axes 1 */
} dit_segment;

/* ------------------------------------------------------------------ host builders
 * Pure host functions: no device, no allocation.  Each is the single source of
 * the table it builds; the forward uses exactly these values. */

/* Packed layout (page "port the MiniMax-H3 omni-modal video+audio DiT", section
 * "Correctness gates": packed layout gated exact).  Writes cu_seqlens[n_segs+1]
 * (running token offsets), cond_idx[N] and doc_id[N]; *n_tokens = N.  Pass NULL
 * for cond_idx/doc_id to get only N and cu_seqlens.  DIT_E_INVALID for a
 * non-positive extent, a segment count outside [1, DIT_MAX_SEGMENTS] or N >= 2^31. */
int dit_pack_layout(const dit_config* cfg, const dit_segment* segs, int n_segs,
                    int32_t* cu_seqlens, int32_t* cond_idx, int32_t* doc_id, int* n_tokens);

/* Per-row rope cache cos/sin [N, rot_dim/2] float32 (page "stream the ORIGINAL
 * bf16 DiT to the device", section "What this enables": built on the host
 * before any kernel).  Integer positions restart at 0 in each segment; the
 * angle of row n, column j is pos_a(n) * inv_freq_a[j'] for the axis block a
 * holding j, inv_freq_a[j'] = 1 / theta^(2j'/axis_dim[a]); cos and sin in fp64,
 * rounded once to float32.  Caller owns both outputs (N * rot_dim/2 floats each). */
int dit_rope_cache_build(const dit_config* cfg, const dit_segment* segs, int n_segs,
                         float* cos_host, float* sin_host);

/* Sinusoidal timestep embedding: out[i, j] = cos(t_i f_j), out[i, dim/2 + j] =
 * sin(t_i f_j), f_j = 10000^(-j/(dim/2)), fp64 math, float32 out [n, dim].
 * The time embedder is one of the fp32 islands of the bf16 stream (page "port
 * the MiniMax-H3 omni-modal video+audio DiT", update "quantized arms land",
 * item 1); the pages print no formula, so this is the standard DiT form,
 * t in [0, 1] unscaled.  t_host [n] float32, out_host [n, dim] caller-owned;
 * DIT_E_INVALID for n < 0, a dim that is not positive and even, or a null
 * pointer. */
int dit_timestep_embedding(const float* t_host, int n, int dim, float* out_host);

/* Time-shifted rectified-flow sigmas (page "port the MiniMax-H3 omni-modal
 * video+audio DiT", update "quantized arms land", item 2: the time-shift
 * sigma schedule; milestone "the whole t2va path composes end to end": shift
 * 12 for video, 3 for audio): s_i = 1 - i/n_steps,
 * sigma_i = shift s_i / (1 + (shift - 1) s_i), i = 0..n_steps (fp64), and
 * dt_i = float32(sigma_{i+1} - sigma_i), i < n_steps.  Either output may be
 * NULL; sigma_host holds n_steps + 1 doubles, dt_host n_steps floats, both
 * caller-owned.  DIT_E_INVALID for n_steps < 1 or a shift that is not
 * positive and finite. */
int dit_sigma_schedule(double shift, int n_steps, double* sigma_host, float* dt_host);

/* ------------------------------------------------------------------ model and staging */

typedef struct dit_model dit_model;

typedef struct dit_weight_view {
  const char* name;     /* weight-name contract below */
  int dtype;            /* DIT_F32 or DIT_BF16 (bf16 as raw uint16 bits) */
  int ndim;
  int64_t shape[4];
  const void* host;     /* host data, row-major, caller-owned */
} dit_weight_view;

typedef struct dit_stage_stats_t {
  int64_t tensors;      /* tensors staged */
  int64_t bytes;        /* device bytes written */
  int64_t direct;       /* staged without conversion */
  int64_t converted;    /* converted on the host (f32 -> bf16 RNE, bf16 -> f32, half swap) */
  int64_t host_peak;    /* largest host conversion buffer held at once (one tensor) */
} dit_stage_stats_t;

/* Bytes of the weight slab for this config (256-byte aligned views), from
 * the config alone, before any weight is read or any memory allocated (page
 * "stream the ORIGINAL bf16 DiT to the device, one tensor at a time", section
 * "What this enables": the manifest first, so the geometry is known before a
 * byte is allocated).  Validates cfg: DIT_E_INVALID names the first field
 * outside what the kernels handle. */
int dit_weight_bytes(const dit_config* cfg, size_t* bytes);

/* Validate cfg and bind a caller-owned device slab of at least dit_weight_bytes
 * that the weights are staged into once and read by every later forward (page
 * "the 2.4B fp32 DiT onto the device, staged once", section "Speed": one
 * staging outside the timed loop).  The handle is library-owned (free with
 * dit_model_destroy); the slab is not, and must outlive the handle.  No
 * device call is made.  DIT_E_INVALID for a bad cfg or a slab smaller than
 * dit_weight_bytes. */
int dit_model_create(const dit_config* cfg, void* weight_slab_dev, size_t slab_bytes,
                     dit_model** out);
void dit_model_destroy(dit_model* m);

/* Stage weights, any subset per call, each name at most once.  Weight-name
 * contract (nn.Linear layout [out, in]; D hidden, F ffn, d cond_dim, c_m the
 * token width of modality m = C*pt*ph*pw or C):
 *   blocks.{b}.adaln.{m}.weight [6D, d]   blocks.{b}.adaln.{m}.bias [6D]
 *   blocks.{b}.attn.qkv.weight  [3D, D]   rows [q_all | k_all | v_all]
 *   blocks.{b}.attn.qkv.bias    [3D]
 *   blocks.{b}.attn.out.weight  [D, D]    blocks.{b}.attn.out.bias [D]
 *   blocks.{b}.mlp.in.weight    [2F, D]   blocks.{b}.mlp.in.bias [2F]
 *   blocks.{b}.mlp.out.weight   [D, F]    blocks.{b}.mlp.out.bias [D]
 *   in.{m}.weight [D, c_m]  in.{m}.bias [D]  out.{m}.weight [c_m, D]  out.{m}.bias [c_m]
 * Block weight matrices are stored in the stream dtype (an f32 view for a bf16
 * stream is rounded to nearest-even on the host through one tensor-sized
 * buffer); biases and the projections in and out stay float32 ("fp32 islands",
 * page "port the MiniMax-H3 omni-modal video+audio DiT", update "quantized arms
 * land").  The fp32 GEMM weights (an fp32 stream's four block matrices and the
 * projections) are staged as the five int8 slices plus per-row exponents the
 * fp32 GEMM consumes (dit_gemm), cut on the host; the AdaLN weights stay as
 * given.  For DIT_MLP_VALUE_GATE the two row halves of mlp.in are swapped so
 * the kernel computes silu(first) * second (page "the 2.4B fp32 DiT onto the
 * device, staged once", section "What moved").  Copies are synchronous on
 * `stream`.  Errors: DIT_E_UNKNOWN_WEIGHT, DIT_E_SHAPE, DIT_E_DTYPE (named),
 * DIT_E_STATE after finalize, DIT_E_INVALID for a repeat. */
int dit_stage_weights(dit_model* m, const dit_weight_view* views, int n, dit_stream_t stream);

/* Close staging.  DIT_E_MISSING_WEIGHT names the first tensor never staged,
 * instead of a forward reading an unwritten slot as zeros (page "port the
 * MiniMax-H3 omni-modal video+audio DiT", update "GGUF arm complete": missing
 * tensors fail by name).  Forward calls need a finalized model (DIT_E_STATE). */
int dit_stage_finalize(dit_model* m);
/* Counters of what staging did -- tensors, device bytes, tensors copied
 * directly and converted on the host, the largest host conversion buffer --
 * so the bound of one tensor of host memory is observable (page "stream the
 * ORIGINAL bf16 DiT to the device, one tensor at a time", sections "What this
 * enables" and "Gates I ran").  out caller-owned; DIT_E_INVALID on null. */
int dit_stage_stats(const dit_model* m, dit_stage_stats_t* out);

/* ------------------------------------------------------------------ batch */

typedef struct dit_batch dit_batch;

/* Device bytes of the batch tables (cu_seqlens, cond_idx, cos, sin, segment
 * table) for these segments: the packed layout of page "port the MiniMax-H3
 * omni-modal video+audio DiT", section "Correctness gates" (cu_seqlens, doc
 * ids), and the per-row rope cache of its section "The device-resident
 * forward (W2b)".  DIT_E_INVALID as dit_pack_layout. */
int dit_batch_bytes(const dit_model* m, const dit_segment* segs, int n_segs, size_t* bytes);

/* Build the batch on the host (layout, rope cache; page "stream the ORIGINAL
 * bf16 DiT to the device", section "What this enables": cos/sin built on the
 * host before any kernel) and copy it into the caller's device buffer
 * `tables_dev` (synchronous on `stream`).  n_cond rows of modulation;
 * cond_modality[c] selects the AdaLN linear of row c (page "port the
 * MiniMax-H3 omni-modal video+audio DiT", section "The device-resident forward
 * (W2b)": indexed AdaLN modulates).  The handle is library-owned; free with
 * dit_batch_destroy.  The buffer must outlive it.  DIT_E_INVALID for a bad
 * segment or modulation row, DIT_E_WORKSPACE for a short buffer,
 * DIT_E_UNSUPPORTED when a GEMM of a forward over this batch would exceed the
 * kernels' 32-bit buffer offsets (checked before any device call). */
int dit_batch_create(const dit_model* m, const dit_segment* segs, int n_segs, int n_cond,
                     const int* cond_modality, void* tables_dev, size_t tables_bytes,
                     dit_stream_t stream, dit_batch** out);
void dit_batch_destroy(dit_batch* b);
/* N, number of segments, longest segment; latent floats of the whole batch
 * (sum over segments of C*T*pt*H*ph*W*pw or C*L; 0 without io).  Any output
 * pointer may be NULL. */
int dit_batch_info(const dit_batch* b, int* n_tokens, int* n_segs, int* max_seqlen,
                   int64_t* latent_floats);
/* Device pointers into the batch tables (for callers driving the op-level calls). */
int dit_batch_tables(const dit_batch* b, const int32_t** cu_seqlens_dev,
                     const int32_t** cond_idx_dev, const float** cos_dev, const float** sin_dev);

/* Workspace bytes that dit_block_forward / dit_forward / dit_denoise_step need:
 * every activation of the forward lives in this caller-owned device buffer,
 * so nothing round-trips through the host (page "port the MiniMax-H3
 * omni-modal video+audio DiT", section "The device-resident forward (W2b)"). */
int dit_workspace_bytes(const dit_model* m, const dit_batch* b, size_t* bytes);

/* ------------------------------------------------------------------ forward */

/* AdaLN table (page "port the MiniMax-H3 omni-modal video+audio DiT",
 * section "The device-resident forward (W2b)": two indexed AdaLN modulates, one
 * linear per modality) of blocks [block0, block0 + n_blocks): mod[b][c][k][D] =
 * (W_ada[b][cond_modality[c]] . cond[c] + bias)[k*D + j], k = shift_msa,
 * scale_msa, gate_msa, shift_mlp, scale_mlp, gate_mlp.  cond_dev [n_cond,
 * cond_dim] float32 (an embedded timestep or a conditioning vector); mod_dev
 * [n_blocks, n_cond, 6, D] float32. */
int dit_modulation(dit_model* m, const dit_batch* b, int block0, int n_blocks,
                   const float* cond_dev, float* mod_dev, dit_stream_t stream);

/* One block on the packed residual stream x_dev [N, D] float32, in place
 * (page "port the MiniMax-H3 omni-modal video+audio DiT", section "The
 * device-resident forward (W2b)"; page "the 2.4B fp32 DiT onto the device,
 * staged once", section "What moved, and onto what").  DIT_E_STATE before
 * finalize, DIT_E_WORKSPACE for a short workspace, DIT_E_INVALID for a block
 * index out of range, DIT_E_HIP for a launch failure.
 * mod_dev [n_cond, 6, D] float32 (this block's rows of dit_modulation).  An
 * fp32 model carries its residual stream in float64 inside the library (here:
 * widened on entry, rounded to float32 once on exit); a bf16 model's is the
 * float32 x_dev itself.  In an fp32 model every GEMM result is still rounded
 * once to float32 before it is used, as dit_gemm returns it: the kernel after
 * each GEMM sums its fp64 split-K partials in split order and adds the bias
 * (the fused kernels change where that happens, not the values). */
int dit_block_forward(dit_model* m, int block, float* x_dev, const float* mod_dev,
                      const dit_batch* b, void* ws_dev, size_t ws_bytes, dit_stream_t stream);

/* The whole forward (page "port the MiniMax-H3 omni-modal video+audio DiT",
 * section "The device-resident forward (W2b)" and update "quantized arms
 * land": fp32 patch projections and output heads around the block stream;
 * page "the 2.4B fp32 DiT onto the device, staged once", section "What moved":
 * 1x1 convolutions as GEMMs on the frame-major activation), asynchronous on
 * `stream`; errors as dit_block_forward.  With io: in_dev holds every segment's latent, segment
 * after segment ([C, T*pt, H*ph, W*pw] or [C, L], float32); out_dev receives
 * the velocities in the same layout.  Without io: in_dev is tokens [N, D]
 * float32 and out_dev the tokens after the last block.  cond_dev as in
 * dit_modulation.  in_dev and out_dev may alias. */
int dit_forward(dit_model* m, const dit_batch* b, const float* in_dev, const float* cond_dev,
                float* out_dev, void* ws_dev, size_t ws_bytes, dit_stream_t stream);

/* One Euler step of the denoise loop, device-resident: v = dit_forward(latents,
 * cond), then latents += dt[modality] * v per segment, in float32 without
 * contraction (euler eta=0 with rf_v_to_x0 reduces to this; page "port the
 * MiniMax-H3 omni-modal video+audio DiT", milestone "the whole t2va path
 * composes end to end").  dt_dev [n_mod] float32.  Requires io. */
int dit_denoise_step(dit_model* m, const dit_batch* b, float* latents_dev, const float* cond_dev,
                     const float* dt_dev, void* ws_dev, size_t ws_bytes, dit_stream_t stream);

/* n_steps consecutive steps with no host round trip (page "port the
 * MiniMax-H3 omni-modal video+audio DiT", section "The device-resident forward
 * (W2b)": the 50-step denoise loop above the block stack stays on the
 * device): step i reads cond_table_dev + i*n_cond*cond_dim and
 * dt_table_dev + i*n_mod (tables built once, e.g. from dit_sigma_schedule and
 * dit_timestep_embedding).  Errors as dit_denoise_step. */
int dit_denoise_loop(dit_model* m, const dit_batch* b, float* latents_dev,
                     const float* cond_table_dev, const float* dt_table_dev, int n_steps,
                     void* ws_dev, size_t ws_bytes, dit_stream_t stream);

/* Guided (classifier-free guidance) denoise loop of a vector-conditioned
 * model, as the music generator runs its DiT (page "the 2.4B fp32 DiT onto
 * the device, staged once", What moved: the conditional and unconditional
 * branches of every step).  The batch holds 2P segments: segment j + P is the
 * unconditional branch of segment j, with the same modality and grid.
 * latents_dev holds the P shared latents, segment after segment (the first
 * half of the batch's latent layout), float32, updated in place.  Step i runs
 * one forward over all 2P segments, both branches of pair j reading latent j,
 * with modulation rows cond_table_dev + i*n_cond*cond_dim, then moves latent j
 * by dt * (v_u + w (v_c - v_u)), dt = dt_table_dev[i*n_mod + modality], each
 * operation rounded to float32 (w = 0: unconditional; w = 1: conditional).
 * Asynchronous on `stream`; no host round trip.  DIT_E_INVALID when the
 * segments do not pair, w is not finite or the model has no io. */
int dit_cfg_denoise_loop(dit_model* m, const dit_batch* b, float* latents_dev,
                         const float* cond_table_dev, const float* dt_table_dev, float w,
                         int n_steps, void* ws_dev, size_t ws_bytes, dit_stream_t stream);

/* ------------------------------------------------------------------ captured forwards
 * dit_forward recorded once as a HIP graph and replayed with one launch, so a
 * forward's few hundred kernel launches cost the host one call (page "the
 * 2.4B fp32 DiT onto the device, staged once", section "Speed": the device
 * loop's fixed per-loop cost measured beside the per-forward slope).  The
 * graph holds the kernels, their arguments and the buffer addresses given at
 * creation: in_dev, cond_dev, out_dev and ws_dev must stay allocated while it
 * lives, and each launch reads their contents as they are then (write new
 * latents into in_dev and launch again).  Creation captures on a stream of
 * its own and launches nothing; it returns the errors of dit_forward, and
 * DIT_E_UNSUPPORTED while per-launch profiling (dit_profile_begin) or
 * DIT_SYNC_CHECK is on.  The caller owns the graph (dit_graph_destroy).
 * Launches of one graph on one stream run in order; two launches of it that
 * overlap in time race on its workspace. */
typedef struct dit_graph dit_graph;
int dit_forward_graph_create(dit_model* m, const dit_batch* b, const float* in_dev, const float* cond_dev,
                             float* out_dev, void* ws_dev, size_t ws_bytes, dit_graph** out);
/* One replay of the captured forward, asynchronous on `stream`; DIT_E_HIP if
 * the launch fails. */
int dit_graph_launch(dit_graph* g, dit_stream_t stream);
/* The number of nodes (kernels and copies) the graph holds. */
int dit_graph_nodes(const dit_graph* g, size_t* nodes);
void dit_graph_destroy(dit_graph* g);

/* ------------------------------------------------------------------ op-level calls
 * The kernels the block is made of, exposed for per-op parity checks and
 * timing: the shared ops the pages compose the block from (page "port the
 * MiniMax-H3 omni-modal video+audio DiT", section "The device-resident forward
 * (W2b)": MatmulBT, RmsNorm, QkvSplit, RopeFromCache, SiluAndMul, Add,
 * DFlashBlockAttention; page "the 2.4B fp32 DiT onto the device", section
 * "What moved": LayerNorm, partial rotary).  dtype arguments are DIT_F32 or
 * DIT_BF16 (bf16 = uint16 bits).  Every pointer is a device pointer the caller
 * owns; calls are asynchronous on `stream`; DIT_E_INVALID for a bad argument,
 * DIT_E_UNSUPPORTED for a shape the kernel does not handle, DIT_E_WORKSPACE
 * for a short workspace. */

/* C[M,N] = A[M,K] . B[N,K]^T + bias[N] (bias may be NULL).  bf16: A, B bf16,
 * fp32 accumulation, C in c_dtype.  DIT_MXFP8: A, B given as bf16, both
 * re-quantized as dit_quantize_mx8 into ws, then multiplied on the scaled fp8
 * matrix cores (K a multiple of 128), C in c_dtype.  DIT_MXFP4: A, B given as
 * bf16, A re-quantized as dit_quantize_mx8 and B as dit_quantize_mx4 into ws,
 * then multiplied on the same matrix cores with B's format FP4 (K a multiple
 * of 128), C in c_dtype.  f32: A, B float32 (K a multiple of 4),
 * each row scaled by a power of two and cut into five 7-bit integer slices,
 * the slice products summed exactly on the int8 matrix cores (pairs whose
 * weight is below 2^-32 of the product dropped), combined in fp64 and
 * rounded once to float32 C.  ws holds B's and A's slices and split-K
 * partials (dit_gemm_workspace_bytes). */
int dit_gemm_workspace_bytes(int dtype, int M, int N, int K, size_t* bytes);
/* Split-K slots of the fp32 GEMM for an [N, K] weight on the current device:
 * the fp64 partials [splits][M][N] that the block's fp32 GEMMs hand to the
 * row kernel after them (the most any column has: the first columns can take
 * fewer splits than the last, to even out the last round of workgroups).
 * Chosen from N, K and the compute-unit count only, so a row's result never
 * depends on M.  dtype must be DIT_F32. */
int dit_gemm_splits(int dtype, int N, int K, int* splits);
/* The same plan as two column groups: columns [0, col_split) of the product
 * in s_lo splits, the rest in s_hi.  A group of one split hands the row kernel
 * after the GEMM finished fp32 values (the bias added, one rounding: 4 bytes
 * per value), any other group its fp64 partials (8 bytes per split and value).
 * dtype must be DIT_F32; no device work.  (Page "the 2.4B fp32 DiT onto the
 * device, staged once", section "What moved, and onto what": the fp32
 * MatmulBT.) */
int dit_gemm_split_groups(int dtype, int N, int K, int* s_lo, int* s_hi, int* col_split);
int dit_gemm(int dtype, int M, int N, int K, const void* A, const void* B, const float* bias,
             void* C, int c_dtype, void* ws, size_t ws_bytes, dit_stream_t stream);

/* The fp32 dit_gemm for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same kernels, same split plan and bit-identical C as
 * dit_gemm(DIT_F32, ...); the scratch (int8 slices of A and B, fp64 split-K
 * partials) lives in a device array built into the library, of
 * dit_gemm_f32_noalloc_limit() bytes (64 MiB) on each device it runs on, held
 * until the process ends.  No allocation, no host synchronisation.  A, B, bias
 * (may be NULL) and C are device pointers the caller owns, C[M,N] float32.
 * Every call on one device shares that device's array: calls that overlap on
 * a device (other streams, or other host threads without ordering) race.
 * DIT_E_WORKSPACE when the shapes need more scratch than the array holds
 * (dit_gemm_workspace_bytes(DIT_F32, ...) gives the need), DIT_E_INVALID /
 * DIT_E_UNSUPPORTED as dit_gemm; nothing is launched then. */
size_t dit_gemm_f32_noalloc_limit(void);
int dit_gemm_f32_noalloc(int M, int N, int K, const float* A, const float* B, const float* bias, float* C,
                         dit_stream_t stream);

/* MXFP8 re-quantization of bf16 rows x [R, K] (K a multiple of 32): codes
 * [R, K] OCP E4M3 bytes, scales [R, K/32] E8M0 bytes.  Per 32 consecutive
 * values the scale is the smallest power of two 2^s with max|v| <= 448 2^s
 * (byte s + 127, s clamped to [-127, 127]), each value v 2^-s rounded to
 * nearest-even E4M3 with its sign; an all-zero block takes byte 0, a block
 * holding a NaN or an Inf byte 255 (NaN) and zero codes.  The pages' low-
 * precision arm is NVFP4 (page "port the MiniMax-H3 omni-modal video+audio
 * DiT", update "NVFP4 arm grounded": FP4 values, an E4M3 scale per 16 and an
 * fp32 global scale); this GPU's matrix cores take MX block scales.  x and
 * codes 16-byte aligned; device pointers; asynchronous. */
int dit_quantize_mx8(int R, int K, const void* x, void* codes, void* scales, dit_stream_t stream);
/* MXFP4 re-quantization of bf16 rows x [R, K] (K a multiple of 32): per 32
 * consecutive values the smallest power-of-two scale 2^s with max|v| <= 6 2^s
 * (E8M0 byte s + 127 into scales [R, K/32]), each v / 2^s rounded to the
 * nearest OCP FP4 E2M1 value, ties to the even mantissa bit (codes [R, K/2],
 * two per byte, the value at even K in the low nibble); an all-zero block
 * takes byte 0, a block holding a NaN or an Inf byte 255 and zero codes
 * (page "port the MiniMax-H3 omni-modal video+audio DiT", update "NVFP4 arm
 * grounded": FP4 values with block scales, here in the OCP MX form).  x and
 * codes 16-byte aligned; asynchronous on `stream`. */
int dit_quantize_mx4(int R, int K, const void* x, void* codes, void* scales, dit_stream_t stream);

/* h[N,D] (dtype) = norm(x[N,D]) * (1 + mod[c][scale_k]) + mod[c][shift_k],
 * c = cond_idx[n]; mod [n_cond, 6, D] f32; which = 0 (msa: shift 0, scale 1) or
 * 1 (mlp: shift 3, scale 4); mod NULL = plain norm.  norm = DIT_NORM_*.  x is
 * x_dtype: DIT_F32, or DIT_F64 (the fp32 stream's residual, dtype DIT_F32). */
int dit_modnorm(int dtype, int norm, float eps, int N, int D, const void* x, int x_dtype,
                const float* mod, int which, const int32_t* cond_idx, void* h, dit_stream_t stream);

/* qkv [N, 3D] (dtype) -> q, k, v head-major [H, N, hd] (dtype); rotate_half
 * RoPE on the first rot dims of q and k from cos/sin [N, rot/2]; v copied. */
int dit_rope_split(int dtype, int N, int H, int hd, int rot, const void* qkv, const float* cos,
                   const float* sin, void* q, void* k, void* v, dit_stream_t stream);

/* o [N, H*hd] (dtype) = per-document softmax(q k^T / sqrt(hd)) v; q, k, v
 * head-major [H, N, hd]; cu_seqlens [n_docs+1] device, max_seqlen its
 * largest gap. */
int dit_attention(int dtype, int N, int H, int hd, int n_docs, const int32_t* cu_seqlens,
                  int max_seqlen, const void* q, const void* k, const void* v, void* o,
                  dit_stream_t stream);

/* m [N, F] (dtype) = silu(u[:, :F]) * u[:, F:]; u [N, 2F] (dtype). */
int dit_silu_gate(int dtype, int N, int F, const void* u, void* m, dit_stream_t stream);

/* x[N,D] += mod[c][gate_k] * a[N,D] f32, c = cond_idx[n]; which 0 (gate 2) or 1
 * (gate 5); x is x_dtype DIT_F32 (fused multiply-add) or DIT_F64 (exact product,
 * one fp64 rounding). */
int dit_gated_residual(int N, int D, void* x, int x_dtype, const float* a, const float* mod, int which,
                       const int32_t* cond_idx, dit_stream_t stream);

/* ------------------------------------------------------------------ diagnostics
 * A failure fails the call, never the process (page "port the MiniMax-H3
 * omni-modal video+audio DiT", section "Serving": a failing runner fails the
 * job, not the process); counters make a launch path observable (page "stream
 * the ORIGINAL bf16 DiT to the device", section "What this enables"). */

/* The calling thread's message of its last failed call (library-owned, valid
 * until that thread's next call). */
const char* dit_last_error(void);
/* Launch counters per kernel family (index order: gemm_bf16, gemm_f32, attention_bf16,
 * attention_f32, modnorm, rope_split, silu_gate, gated_residual, adaln, patch_in,
 * patch_out, euler, gemm_f32_reduce, convert, resid_norm_slice, silu_slice); n_max entries written; returns DIT_OK. */
int dit_counters(int64_t* out, int n_max);
void dit_counters_reset(void);

/* Per-kernel timing, for the device-side timing protocol of page "the 2.4B
 * fp32 DiT onto the device, staged once", section "Speed" (only the forward
 * loop timed).  Between dit_profile_begin and dit_profile_end every
 * launch records a HIP event pair around itself on its own stream (a few
 * microseconds of host time per launch).  dit_profile_end waits for those
 * events and writes, per kernel family (index order as dit_counters), the
 * number of launches and their summed device time in milliseconds. */
int dit_profile_begin(void);
int dit_profile_end(int64_t* counts, double* total_ms, int n_max);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H */

/*
 * cc3d.h -- chunked causal 3-D convolution decode on AMD Instinct MI355X (gfx950).
 *
 * A video decoder's causal conv stack, streamed in temporal chunks.  Each conv
 * keeps the last k_t-1 frames of its own input as state, so a video decoded
 * chunk by chunk equals one pass over the whole video:
 *   - LightX2V blog "SwiftVR Inference Optimization: From One GPU to Causal Chunk
 *     Parallelism", section "From Pixels to Latents and Back" (every layer keeps
 *     boundary features across chunks) and section "ReAE: Causal Halo Exchange"
 *     (a chunk needs only the previous chunk's trailing input frames at each
 *     layer; the video's first chunk takes zeros as history);
 *   - same page, section "TemporalGrow: Compute Before Spatial Upsampling"
 *     (nearest 2x upsampling followed by a spatial conv; per-position ops commute
 *     with the upsample);
 *   - AWS/Synthesia digest (sysdesign-wiki), "Key takeaways" 1: decode is chunked
 *     along time, one latent frame giving four pixel frames.
 * The interface follows the stateful causal video module of the PyPI page
 * "pixtreme-infer-cda-vsr 0.10.3", sections "CUDA Graph inference" and "Frame,
 * state and stream requirements": one instance per shape and precision, two
 * state buffers used alternately, reset that clears state without
 * reallocating, validation of every argument before any state changes, all
 * work enqueued on the caller's stream, and open that fails cleanly.
 *
 * Definition of one conv (X~ = the k_t-1 history frames followed by the input
 * sequence; spatial indices outside the image read 0; ph=(k_h-1)/2, pw=(k_w-1)/2):
 *   Y[o,t,h,w] = B[o] + sum_{c,a,b,d} W[o,c,a,b,d] * X~[c, t+a, h+b-ph, w+d-pw]
 * History is zeros (CC3D_TPAD_ZERO) or copies of the first frame
 * (CC3D_TPAD_REPLICATE).  With up_s = 2 the conv reads the nearest-upsampled
 * input U[h,w] = X[h/2, w/2]; with up_t = 2 it reads the input grown in time on
 * non-first frames: V[0] = X[0], V[2j-1] = V[2j] = X[j] (or, under the aligned
 * growth rule below, every frame: V[2j] = V[2j+1] = X[j]).  The epilogue adds the
 * bias and an optional residual, and can store SiLU(RMSNorm(.)) of the result:
 *   RMSNorm(v)_c = gamma_c * v_c / sqrt(mean_c v^2 + eps),  SiLU(z) = z / (1 + e^-z).
 *
 * Layout.  Every activation is channels-last, one video: [T][H][W][C],
 * contiguous, element type = the plan's dtype (bfloat16 bits or float32).
 * Weights are given in PyTorch order [Cout][Cin][k_t][k_h][k_w].  bias and gamma
 * are float32.  All pointers passed to this library are device pointers on the
 * plan's device unless stated otherwise; the library never retains a caller's
 * buffer beyond the call that takes it (weights are copied and repacked).
 *
 * Errors.  Every entry point returns a cc3d_status.  On an error nothing is
 * enqueued and no state or output is modified; cc3d_last_error() returns a
 * thread-local message naming the observed and the accepted value.
 *
 * Streams.  Calls enqueue work on the given HIP stream (hipStream_t passed as
 * void*; NULL = the null stream) and return without synchronising the host.
 * Inputs must stay alive until that work completes.  One plan and one state
 * must not be used by two calls at once (a plan owns its intermediate buffers).
 *
 * Graphs (CDA-VSR page, "CUDA Graph inference").  cc3d_forward_chunk and
 * cc3d_reset only launch kernels on the stream (no allocation, no host
 * synchronisation, no memset nodes) and may be captured into a HIP graph, with
 * profiling off.  Which rule a chunk takes (first chunk or not) is decided from
 * cache_in->frames_seen when the call is made, so a captured call replays that
 * rule: run the video's first chunk eagerly, then replay captured chunks.
 */
#ifndef CC3D_H
#define CC3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CC3D_VERSION 105 /* 1.0.5: strided convs (the encoder side) */

typedef enum {
    CC3D_OK = 0,
    CC3D_EINVAL = 1,  /* null or out-of-range argument */
    CC3D_ESHAPE = 2,  /* shape not accepted (sizes, kernel, channel alignment) */
    CC3D_EDTYPE = 3,  /* element type not accepted */
    CC3D_ESTATE = 4,  /* state misuse: aliasing caches, negative frame count */
    CC3D_ENOMEM = 5,  /* device allocation failed (everything partial released) */
    CC3D_EDEVICE = 6  /* HIP runtime error, or pointer/stream on another device */
} cc3d_status;

typedef enum { CC3D_F32 = 0, CC3D_BF16 = 1 } cc3d_dtype;

typedef enum {
    CC3D_TPAD_REPLICATE = 0, /* history = copies of the first frame */
    CC3D_TPAD_ZERO = 1       /* history = zeros (the MemoryBlock rule) */
} cc3d_tpad;

/* Temporal growth of the video's first chunk at every up_t = 2 conv.
 * CC3D_GROW_ONCE: its first frame is not doubled (T -> 2T-1; later chunks 2T).
 * CC3D_GROW_ALIGNED: every frame is doubled (T -> 2T), as for later chunks.  This
 * is the first chunk of the SwiftVR page ("From Pixels to Latents and Back"):
 * the reader takes 28 frames (7 latents, 4 frames each) and drops the 3 frames
 * used for temporal alignment after decoding.  With two up_t = 2 stages and
 * replicate history, the aligned video is the ONCE video with its first frame
 * three extra times in front, so dropping y's first 3 frames of the first chunk
 * gives the ONCE video.  The caller drops them (y holds all 2T.. frames). */
typedef enum { CC3D_GROW_ONCE = 0, CC3D_GROW_ALIGNED = 1 } cc3d_grow;

/* ----------------------------------------------------------------------------
 * Single conv plan (the causal conv3d plan).
 * y = conv(x) + bias [+ residual]; with CC3D_EPI_ACT, y = SiLU(RMSNorm(that)).
 */
#define CC3D_EPI_NONE 0
#define CC3D_EPI_RESIDUAL 1 /* forward_chunk's residual (shape of y) is added */
#define CC3D_EPI_ACT 2      /* store SiLU(RMSNorm(result)) using gamma [Cout] */
#define CC3D_EPI_U8 4       /* store y as 8-bit codes (see "8-bit output" below) */

/* 8-bit output (CC3D_EPI_U8, or out_u8 on the stack op that writes y): the
 * output is delivered as uint8 codes instead of the plan dtype, as a video
 * decoder hands RGB frames to an encoder (LightX2V blog "SwiftVR Inference
 * Optimization ...", section "Other Engineering Optimizations": the output is
 * converted to uint8 on the GPU, halving the payload sent to the host).  The page
 * does not state the mapping; the one used here is the usual one for a decoder
 * whose output range is [-1, 1]:
 *   q = rint(clamp((v + 1) * 127.5, 0, 255))   (rint: round half to even)
 * taken from the fp32 result v (conv + bias + residual) before any rounding to
 * the plan dtype.  bf16 plans only, and not for 3x3 spatial convs whose output
 * channels are split into 96- or 128-channel blocks (cout in 65..128, or a
 * multiple of 96 or 128 above that; CC3D_ESHAPE); it cannot be combined with
 * an act. */

typedef struct {
    int cin, cout;        /* channels; bf16 plans need cin % 8 == 0 */
    int kt, kh, kw;       /* 1 <= k <= 3; kh, kw odd (spatial "same" padding) */
    int h_in, w_in;       /* input frame size (before upsampling) */
    int up_s, up_t;       /* nearest upsample folded into the conv: 1 or 2 each */
    int max_chunk_t;      /* largest t_chunk forward_chunk accepts (>= 1) */
    int dtype;            /* cc3d_dtype */
    int tpad;             /* cc3d_tpad */
    int epilogue;         /* CC3D_EPI_* flags */
    float eps;            /* RMSNorm epsilon (CC3D_EPI_ACT) */
    int grow;             /* cc3d_grow (first chunk at up_t = 2) */
    int fold_upsample;    /* 1: phase-folded upsample conv where it applies (see below) */
    int stride_s, stride_t; /* strided conv (see "Strided convs" below): 1 or 2 each;
                               0 reads as 1 */
} cc3d_conv_desc;

typedef struct cc3d_plan cc3d_plan;

/* Causal conv state: the caches of every conv in a plan, plus the number of
 * input frames consumed.  The caller allocates `arena` (cc3d_state_bytes bytes of
 * device memory, 256-byte aligned) twice and alternates them as cache_in /
 * cache_out across chunks; copying an arena and frames_seen checkpoints the
 * stream exactly. */
typedef struct {
    void* arena;
    int64_t frames_seen; /* 0 after reset: the next chunk is the video's first */
} cc3d_state;

/* Create a plan for one conv.  w: device, dtype elements, [cout][cin][kt][kh][kw];
 * bias: device float32 [cout] or NULL (zero); gamma: device float32 [cout],
 * required with CC3D_EPI_ACT, else ignored.  Weights are copied and repacked on
 * `stream`; the call synchronises that stream once before returning, so the
 * caller may free w afterwards.  On failure *out is NULL and nothing leaks. */
cc3d_status cc3d_plan_create(const cc3d_conv_desc* desc, const void* w, const float* bias,
                             const float* gamma, void* stream, cc3d_plan** out);

/* ----------------------------------------------------------------------------
 * Stack plan: an ordered list of ops run on every chunk.
 * Tensors live in slots: CC3D_SLOT_X = the chunk input x, CC3D_SLOT_Y = the
 * output y, CC3D_SLOT_AUX = forward_chunk's `residual` argument, slots 3.. are
 * intermediates owned by the plan.  A slot's channel count, frame size and frame
 * count follow from the op that writes it; every reader must agree.
 */
#define CC3D_SLOT_NONE (-1)
#define CC3D_SLOT_X 0
#define CC3D_SLOT_Y 1
#define CC3D_SLOT_AUX 2
#define CC3D_MAX_SLOTS 64
#define CC3D_MAX_OPS 256

typedef enum {
    CC3D_OP_CONV = 0,    /* causal conv of src (+ bias, + res) */
    CC3D_OP_NORM_ACT = 1 /* v = src (+ res); out = v; act_out = SiLU(RMSNorm(v)) */
} cc3d_op_kind;

typedef struct {
    int kind;          /* cc3d_op_kind */
    int cout;          /* CONV: output channels; NORM_ACT: ignored (= src channels) */
    int kt, kh, kw;    /* CONV only */
    int up_s, up_t;    /* CONV only: 1 or 2 */
    int tpad;          /* CONV only: cc3d_tpad */
    int src;           /* input slot */
    int res;           /* residual slot (same shape as the result) or CC3D_SLOT_NONE */
    int out;           /* slot for the result v, or CC3D_SLOT_NONE */
    int act_out;       /* slot for SiLU(RMSNorm(v)), or CC3D_SLOT_NONE */
    const void* w;     /* CONV: device weights [cout][cin][kt][kh][kw], plan dtype */
    const float* bias; /* CONV: device float32 [cout] or NULL */
    const float* gamma;/* device float32 [channels of v]; required when act_out is set */
    int out_u8;        /* CONV writing CC3D_SLOT_Y only: 1 = y as 8-bit codes (CC3D_EPI_U8) */
    int stride_s, stride_t; /* CONV only: 1 or 2 each (0 reads as 1); see "Strided convs" */
} cc3d_op_desc;

typedef struct {
    int dtype;          /* cc3d_dtype for every tensor of the stack */
    int cin, h, w;      /* chunk input x: [t][h][w][cin] */
    int max_chunk_t;    /* largest t_chunk accepted */
    float eps;          /* RMSNorm epsilon for every act */
    int n_ops;          /* 1 .. CC3D_MAX_OPS */
    const cc3d_op_desc* ops;
    int grow;           /* cc3d_grow for every up_t = 2 conv of the stack */
    int batch_from;     /* frame batching (see below): first op of the group */
    int frame_batch;    /* frames per batch of the group input; 0 = off */
    int fold_upsample;  /* 1: phase-folded upsample convs where they apply (see below) */
} cc3d_stack_desc;

/* Phase-folded upsample convs (fold_upsample = 1; bf16, 3x3 spatial kernels with
 * up_s = 2 whose output channels are taken in 96-channel blocks, not with 8-bit
 * output).  Nearest 2x upsampling followed by a 3x3 conv is, at each output
 * phase (y & 1, x & 1), a 2x2 conv of the source image (the taps that read the
 * same source pixel are summed first; the SwiftVR page's "compute once, then
 * copy" reasoning, section "TemporalGrow: Compute Before Spatial Upsampling",
 * applied to the weights).  Where the conv also doubles time (up_t = 2), the
 * temporal taps that read the same input frame are summed the same way (two of
 * the three taps of almost every output frame).  Each folded weight is kept as a
 * bf16 hi/lo pair (about 2^-17 relative), so the result equals the conv up to
 * fp32 rounding while the executed MFMA work is 7/9 of the definition's (about
 * 16/27 with time doubled); profiling still reports the definition's
 * (algorithmic) FLOP. */

/* Frame batching (LightX2V blog "SwiftVR Inference Optimization ...", section
 * "ReAE Frame Batching": a small batch of frames passes through a whole group of
 * consecutive layers before the next batch starts, so only that batch's
 * intermediate features are held, and every batch writes its part of one output
 * buffer; causal layers keep their state rules).  With frame_batch > 0, ops
 * batch_from .. n_ops-1 run once per batch of frame_batch frames of the group
 * input -- the slots the group reads from ops before it (or x), which must all
 * have the same frame count -- and the slots those ops write hold one batch
 * (frames, and device memory, per batch instead of per chunk).  Each conv of the
 * group carries its cache from batch to batch.  The output equals the
 * whole-chunk run bit for bit.  The group must write y and must not read the
 * residual argument or write a slot written before it; cc3d_slot_shape and
 * cc3d_slot_read reject the group's slots (CC3D_EINVAL). */

/* Strided convs (stride_s, stride_t = 2; the encoder side: the SwiftVR page,
 * "ReAE: Causal Halo Exchange", puts the ReAE encoder under the decoder's
 * causal-state rule, and "From Pixels to Latents and Back" has it map the video
 * to latents; the page prints no encoder layer).  stride_s = 2: output pixel
 * (y, x) is the conv centred on input pixel (2y, 2x), zero padding (k-1)/2, so
 * an H x W input gives ceil(H/2) x ceil(W/2) (PyTorch's stride convention).
 * stride_t = 2: the outputs are those whose current frame is an input frame
 * tau = phase (mod 2), counted over the whole video; phase 0 (CC3D_GROW_ONCE:
 * the first frame on its own, 1 + 2n frames -> 1 + n) or 1 (CC3D_GROW_ALIGNED:
 * every output takes two new frames, 2n -> n).  The cache is the last kt-1
 * input frames, as for any conv.  Chunks must keep the count whole at every
 * strided layer: with phase 0 the video's first chunk brings an odd number of
 * frames to that layer and later chunks an even number; with phase 1 every
 * chunk an even number (forward_chunk, cc3d_output_shape: CC3D_ESHAPE
 * otherwise).  Not with up_s = 2 (stride_s) or up_t = 2 (stride_t) on the same
 * conv, not inside a frame-batched group, not with 8-bit output; bf16 strided
 * convs take kh = kw in {1, 3}. */

/* Create a stack plan (same ownership, failure and synchronisation rules as
 * cc3d_plan_create).  The plan allocates its intermediate slots for
 * max_chunk_t input frames. */
cc3d_status cc3d_stack_plan_create(const cc3d_stack_desc* desc, void* stream, cc3d_plan** out);

/* Free a plan (NULL is accepted).  The caller must first make sure no work that
 * uses the plan is still running. */
void cc3d_plan_destroy(cc3d_plan* plan);

/* Bytes of one state arena (>= 256). */
size_t cc3d_state_bytes(const cc3d_plan* plan);

/* Device bytes the plan holds (packed weights and intermediates). */
size_t cc3d_plan_device_bytes(const cc3d_plan* plan);

/* Bytes per element of y: 1 with 8-bit output, else that of the plan dtype
 * (0 for an invalid plan). */
int cc3d_output_elem_bytes(const cc3d_plan* plan);

/* Output shape of one forward_chunk: y is [*t][*h][*w][*c].  first != 0 for the
 * video's first chunk (frames grow by 2t-1 instead of 2t at each up_t = 2, unless
 * the plan uses CC3D_GROW_ALIGNED; strided convs: see "Strided convs").
 * CC3D_ESHAPE when t_chunk leaves a strided conv a fractional frame count. */
cc3d_status cc3d_output_shape(const cc3d_plan* plan, int t_chunk, int first, int* c, int* t,
                              int* h, int* w);

/* Reset `state` to the start of a video: frames_seen = 0 and the arena cleared
 * (a fill kernel on `stream`; no allocation).  The next chunk takes the history
 * rule (zeros or copies of its first frame). */
cc3d_status cc3d_reset(const cc3d_plan* plan, cc3d_state* state, void* stream);

/* Decode one chunk.
 * x        : device [t_chunk][h][w][cin], plan dtype; 1 <= t_chunk <= max_chunk_t
 * cache_in : state before the chunk (read only; its arena is not modified)
 * cache_out: receives the state after the chunk: its arena is overwritten and
 *            frames_seen = cache_in->frames_seen + t_chunk.  cache_out->arena
 *            must differ from cache_in->arena (CC3D_ESTATE otherwise).
 * residual : device tensor for CC3D_SLOT_AUX (a single-conv plan with
 *            CC3D_EPI_RESIDUAL: shape of y), else must be NULL
 * y        : device output, shape from cc3d_output_shape; must not overlap x
 * x, y, residual and both arenas must be 16-byte aligned (CC3D_EINVAL otherwise).
 * A t_chunk that would leave a strided conv a fractional frame count is refused
 * (CC3D_ESHAPE; see "Strided convs"), like every other check before any work.
 * Returns without synchronising; later calls never modify a returned y. */
cc3d_status cc3d_forward_chunk(const cc3d_plan* plan, const void* x, int t_chunk,
                               const cc3d_state* cache_in, cc3d_state* cache_out,
                               const void* residual, void* y, void* stream);

/* One conv chunk that allocates no device memory, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments and result as cc3d_plan_create(desc, w,
 * bias, gamma) followed by cc3d_forward_chunk(plan, x, t_chunk, cache_in,
 * cache_out, residual, y) -- the same validation, kernels and output, bit for
 * bit -- but the weights are repacked on every call, on `stream`, into a
 * fixed scratch array of CC3D_NOALLOC_SCRATCH_BYTES that the library holds
 * on each device it runs on until the process ends (with the intermediate of
 * an act the conv's kernel does not fuse, and copies of bias and gamma).  A
 * conv whose repacked weights and intermediates do not fit is rejected
 * (CC3D_ENOMEM) before any device work.  The state arenas are the caller's,
 * of cc3d_state_bytes of a plan made from the same descriptor (e.g. at set-up).
 * No call synchronises or allocates; the first call on a device (or the first
 * plan creation there) looks the scratch's address up.  Every call on a device
 * shares that device's scratch: calls that overlap on one device (two streams,
 * or two host threads) race and must be ordered by the caller.  Nothing in
 * the scratch needs to start at zero (every byte a call reads it first
 * writes). */
#define CC3D_NOALLOC_SCRATCH_BYTES (64u << 20)
cc3d_status cc3d_conv_forward_noalloc(const cc3d_conv_desc* desc, const void* w, const float* bias,
                                      const float* gamma, const void* x, int t_chunk,
                                      const cc3d_state* cache_in, cc3d_state* cache_out,
                                      const void* residual, void* y, void* stream);

/* Channels-first <-> channels-last copies of one video tensor (the boundary
 * between a [C][T][H][W] caller and this library's [T][H][W][C]); elem_bytes is
 * 2 or 4.  Enqueued on stream; src and dst must not overlap. */
cc3d_status cc3d_to_channels_last(const void* src_cthw, void* dst_thwc, int c, int t, int h,
                                  int w, int elem_bytes, void* stream);
cc3d_status cc3d_to_channels_first(const void* src_thwc, void* dst_cthw, int c, int t, int h,
                                   int w, int elem_bytes, void* stream);

/* Intermediate slots (index >= 3) hold what the last forward_chunk wrote, until
 * the next forward_chunk on the plan.  cc3d_slot_shape gives a slot's shape for a
 * chunk of t_chunk input frames (also for CC3D_SLOT_AUX, the shape forward_chunk's
 * residual must have, when the plan reads one); cc3d_slot_read copies an
 * intermediate slot's contents for that chunk (dst: device, at least c*t*h*w
 * elements of the plan dtype) on stream.  Used to inspect every layer of a stack
 * (layer-wise parity checks).  CC3D_ESHAPE for a t_chunk a strided conv of the
 * plan cannot take. */
cc3d_status cc3d_slot_shape(const cc3d_plan* plan, int slot, int t_chunk, int first, int* c, int* t,
                            int* h, int* w);
cc3d_status cc3d_slot_read(const cc3d_plan* plan, int slot, int t_chunk, int first, void* dst,
                           size_t dst_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * Live kernel timing.  With profiling on, forward_chunk records a HIP event pair
 * on its stream around every launch; cc3d_profile_read waits for the recorded
 * events and returns the totals for one op and one part of it:
 *   part 0 = the op's main kernel (the conv, or the norm of a NORM_ACT op)
 *   part 1 = the separate norm pass of a conv whose act is not fused
 *   part 2 = the cache update of a conv
 * Algorithmic counts per launch: a conv does 2*Cin*Cout*kt*kh*kw FLOP per output
 * voxel and moves its input window (T_in+kt-1 frames read once), its weights
 * and its outputs (+ residual) once; a norm pass reads and writes C values per
 * position; a cache update reads and writes its kt-1 frames.
 */
typedef struct {
    char kernel[64];  /* kernel family, e.g. "conv_bf16_up2_k3_n96" ("" = no such launch) */
    int64_t launches; /* launches recorded since profiling was switched on */
    double total_ms;  /* summed event time of those launches */
    double flops;     /* algorithmic FLOP of those launches */
    double bytes;     /* algorithmic HBM bytes of those launches */
} cc3d_op_profile;

/* Switch event timing on (1) or off (0); either way the counters restart. */
cc3d_status cc3d_profile_enable(cc3d_plan* plan, int enable);

/* Number of ops of a plan (a single-conv plan has 1). */
int cc3d_plan_num_ops(const cc3d_plan* plan);

/* Totals for (op, part); synchronises on the recorded events (host wait). */
cc3d_status cc3d_profile_read(const cc3d_plan* plan, int op, int part, cc3d_op_profile* out);

/* Thread-local description of the last error on this thread ("" if none). */
const char* cc3d_last_error(void);

/* CC3D_VERSION of the library. */
int cc3d_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CC3D_H */

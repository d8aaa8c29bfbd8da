/*
 * ltxattn.h -- C ABI of the per-block attention set of the LTX-2 joint
 * video+audio DiT, for AMD Instinct MI355X (gfx950).
 *
 * Every block of the joint DiT runs four softmax attentions,
 * O = softmax(Q K^T / sqrt(D)) V, over two token streams (TensorRT-LLM
 * PR #16228 "LTX-2: replicate audio stream across Ulysses ranks by
 * default", section "Description", names them and their pairing):
 *
 *   LTXATTN_VIDEO_SELF  video queries over video keys/values (the long one:
 *                       15360 tokens for a 768x1280x121 clip)
 *   LTXATTN_AUDIO_SELF  audio queries over audio keys/values (126 tokens)
 *   LTXATTN_A2V         video queries over audio keys/values
 *   LTXATTN_V2A         audio queries over video keys/values
 *
 * The audio stream is padded (same PR, "Description": audio is padded to a
 * multiple of the sequence-parallel degree), so the caller passes the
 * number of valid audio keys; audio key rows at or beyond it get weight
 * exactly zero and are never read.  Padded audio query rows are computed
 * like any other row.  Q and K arrive normalised and rotary-embedded (the
 * context-parallel DiT of TensorRT-Model-Connect PR #1586 all-gathers keys
 * after those steps); a caller may instead hand over the raw Q and K with
 * the parameters of those two steps (ltxattn_qk_prologue), and the library
 * applies them on the way in.
 *
 * Precision: bf16 inputs and outputs with fp32 accumulation and fp32
 * softmax statistics (the DiT of PR #1586 keeps the network in bf16 with
 * fp32 for norms and similar steps).  Outputs are rounded to bf16 to nearest
 * even.
 *
 * Layout: every tensor is [B, S, H, D] bf16 with D contiguous (stride 1)
 * and explicit batch/sequence/head strides in elements, so both the packed
 * token-major layout and [B, H, S, D] are accepted.
 *
 * Ownership and execution: the caller allocates and owns every tensor and
 * the stream; the library keeps no pointer past the call.  A call only
 * enqueues work on the given HIP stream and returns; there is no host
 * synchronisation inside.  A handle owns its device workspace and is not
 * thread-safe: use one handle per stream.
 *
 * Errors: every entry point returns an int status (LTXATTN_OK = 0).  All
 * arguments are validated before anything is enqueued, so a rejected call
 * has no effect on the device.  Nothing is printed, no exception crosses
 * the ABI and the library never aborts the process.
 */
#ifndef LTXATTN_H
#define LTXATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LTXATTN_OK               0
#define LTXATTN_ERR_INVALID_ARG (-1) /* null/misaligned pointer, bad stride, size out of range,
                                        output overlapping another tensor */
#define LTXATTN_ERR_UNSUPPORTED (-2) /* head_dim not 64 or 128, heads < 1, tensor too large
                                        for 32-bit buffer offsets, split parts that would not
                                        fit the workspace, a prologue on a handle created
                                        without its workspace (or on the allocation-free call) */
#define LTXATTN_ERR_HIP         (-3) /* a HIP call or kernel launch failed; see
                                        ltxattn_last_hip_error */
#define LTXATTN_ERR_OOM         (-4) /* device workspace allocation failed */
#define LTXATTN_ERR_SCRATCH     (-5) /* ltxattn_block_attention_noalloc: the call's split parts
                                        need more than its static scratch */

/* Attention kinds (index into ltxattn_block_io.attn). */
enum {
    LTXATTN_VIDEO_SELF = 0,
    LTXATTN_AUDIO_SELF = 1,
    LTXATTN_A2V = 2,
    LTXATTN_V2A = 3,
    LTXATTN_NUM_KINDS = 4
};

typedef struct ltxattn_handle ltxattn_handle;

/* Fixed at create time.  heads and head_dim are shared by all four
 * attentions.  The max_* capacities bound every later call.  The handle's
 * device workspace of split work items (the key-range parts of v2a and of
 * an incomplete last round of video self-attention, in separate regions)
 * is sized by the device's compute units: 384 rows of head_dim + 2 floats
 * per CU, 51 MB at head_dim 128 on a 256-CU MI355X. */
typedef struct {
    int32_t device;        /* HIP device ordinal the handle and its kernels use */
    int32_t heads;         /* H >= 1 */
    int32_t head_dim;      /* D, 64 or 128 */
    int32_t max_batch;     /* >= 1 */
    int32_t max_video_len; /* >= 1, video tokens */
    int32_t max_audio_len; /* >= 1, audio buffer rows (padded length) */
    int32_t qk_prologue;   /* 1: the handle also holds the workspace of the keys of the
                              QK-norm + rotary prologue (two video-sized and two
                              audio-sized bf16 key tensors at the capacities); 0: calls
                              with a prologue are refused */
} ltxattn_config;

/* One bf16 tensor [B, S, H, D], D contiguous.  data is a device pointer,
 * 16-byte aligned; strides are in elements and must be multiples of 8 with
 * stride_s >= D and stride_h >= D.  An output's distinct (b, s, h) rows must
 * not share memory (inputs may, e.g. a batch stride of 0).  Caller-owned. */
typedef struct {
    void *data;
    int64_t stride_b, stride_s, stride_h;
} ltxattn_tensor;

/* Rotary pairings of the QK-norm + rotary prologue. */
enum {
    LTXATTN_ROPE_HALF = 0,        /* channel i pairs with channel i + D/2 */
    LTXATTN_ROPE_INTERLEAVED = 1  /* channel 2i pairs with channel 2i + 1 */
};

/* Optional QK-norm + rotary prologue of one attention (q_weight == NULL:
 * none; the keys and queries of the joint DiT are normed and rotated before
 * attention, with fp32 norm and RoPE islands in a bf16 network, PR #1586,
 * the commit onboarding LTX-2.5; its RoPE tables are data per latent grid,
 * same PR, "The DiT plan serves both grids").  The pages give no formulas;
 * what is computed, for every (batch, token s, head) row x of q (and of k,
 * with the k parameters):
 *   r   = 1 / sqrt(mean over the D channels of x^2 + eps)
 *   y_d = x_d * r * weight[d]                     (RMS norm, per head)
 *   for every pair i < D/2 of channels (a, c):
 *     out_a = y_a * cos[s][i] - y_c * sin[s][i]
 *     out_c = y_a * sin[s][i] + y_c * cos[s][i]   (rotation)
 * in fp32, rounded to bf16 before the attention reads it.  The weights are
 * fp32 [D]; the tables fp32 [rows][D/2], row-major, one row per token of
 * that tensor (every buffer row: video_len or audio_len rows); all six
 * pointers are device pointers, 16-byte aligned, and must be given when
 * q_weight is.  eps > 0.  Q is normed and rotated as the attention kernels
 * load it; K by a pass that writes the prepared keys into the handle's
 * workspace (kinds that name the same K tensor and the same k parameters
 * share that pass). */
typedef struct {
    const float *q_weight, *k_weight;
    const float *q_cos, *q_sin;
    const float *k_cos, *k_sin;
    float eps;
    int32_t pairing;   /* LTXATTN_ROPE_HALF or LTXATTN_ROPE_INTERLEAVED */
} ltxattn_qk_prologue;

/* One attention's tensors.  gate is optional (gate.data == NULL: none):
 * a per-channel output gate of o's shape and layout rules, bf16; when given,
 * o = gate * softmax(Q K^T / sqrt(D)) V elementwise, the product taken in
 * fp32 before the output's rounding to bf16.  PR #1586 names gated attention
 * among the DiT's parts without its formula: the gate values, already
 * activated, come from the caller.  A gate may alias inputs, not outputs. */
typedef struct {
    ltxattn_tensor q, k, v, o;
    ltxattn_tensor gate;
    ltxattn_qk_prologue prologue;
} ltxattn_attn_io;

/* One block call.  Row counts by kind:
 *   VIDEO_SELF: q, k, v, o have video_len rows;
 *   AUDIO_SELF: q, k, v, o have audio_len rows;
 *   A2V: q, o have video_len rows, k, v have audio_len rows;
 *   V2A: q, o have audio_len rows, k, v have video_len rows.
 * gate, when given, has the rows of o.
 * Keys j >= audio_kv_len are masked whenever K/V are audio (AUDIO_SELF, A2V);
 * 1 <= audio_kv_len <= audio_len.  An entry with o.data == NULL is skipped.
 * The four entries may share input tensors (the usual case: one video and
 * one audio Q/K/V triple); an output may not overlap any input or other
 * output of the call. */
typedef struct {
    int32_t batch;
    int32_t video_len;
    int32_t audio_len;
    int32_t audio_kv_len;
    ltxattn_attn_io attn[LTXATTN_NUM_KINDS];
} ltxattn_block_io;

/* Create a handle on cfg->device and allocate its workspace.
 * On success *out receives the handle; on failure *out is set to NULL.
 * Errors: INVALID_ARG (null pointer, capacity < 1, device out of range),
 * UNSUPPORTED (head_dim, heads), HIP, OOM. */
int ltxattn_create(const ltxattn_config *cfg, ltxattn_handle **out);

/* Enqueue the block's attentions on hip_stream (a hipStream_t; NULL is the
 * default stream), in the fixed order VIDEO_SELF, V2A, A2V, AUDIO_SELF.
 * V2A runs as a split-KV pass writing fp32 partial results and softmax
 * statistics into the handle's workspace, then a combine pass that merges
 * them by log-sum-exp in a fixed order (VIDEO_SELF does the same for the
 * query tiles of an incomplete last round, when there is one); the other
 * work writes bf16 O directly.  Results are bit-identical from run to run.
 * Every argument is checked, and every kind's launch and workspace planned,
 * before anything is enqueued.
 * Errors: INVALID_ARG, UNSUPPORTED (both before any launch), HIP. */
int ltxattn_block_attention(ltxattn_handle *h, const ltxattn_block_io *io, void *hip_stream);

/* The same block call with the audio side running beside video
 * self-attention: VIDEO_SELF is enqueued on hip_stream, V2A, A2V and
 * AUDIO_SELF (same order) on a stream the handle owns, which is forked from
 * hip_stream at the start of the call and joined back into it at the end
 * (HIP events; no host synchronisation).  Work enqueued on hip_stream after
 * the call therefore sees all four outputs, and the call can be captured
 * into a HIP graph from hip_stream.  Outputs are bit-identical to
 * ltxattn_block_attention's (the same kernels; only video self-attention
 * and v2a use the workspace, each its own region).  Calls on one handle
 * must not overlap each other, as for ltxattn_block_attention.  The audio side is a few percent of a
 * block (PR #16228, "Description"); whether running it beside video
 * self-attention shortens the block depends on how much of the device the
 * video kernel leaves free.
 * Errors: as ltxattn_block_attention. */
int ltxattn_block_attention_overlap(ltxattn_handle *h, const ltxattn_block_io *io, void *hip_stream);

/* The block call of ltxattn_block_attention without a handle and without
 * allocating anything, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  cfg gives the device and the sizes the call is checked
 * against, as for ltxattn_create.  The same kernels run in the same order on
 * hip_stream and the outputs are bit-identical to ltxattn_block_attention's;
 * the split parts of video self-attention's last round and of v2a go to a
 * static scratch array of 64 MiB per device instead of a handle's workspace
 * (each device the library runs on holds its copy until the process ends).
 * A call needs (rows of split parts) x (head_dim + 2) x 4 bytes of it, at
 * most 384 rows per compute unit: 51 MB at head_dim 128 on a 256-CU MI355X,
 * so every request fits there; a request that would not fit is rejected
 * with LTXATTN_ERR_SCRATCH before anything is enqueued.  Nothing in the
 * scratch needs to start at zero: every part writes all its rows before the
 * combine kernel reads them.  All calls on one device share its scratch, so
 * calls whose work overlaps in time on one device (other streams, other
 * threads) race and must be avoided.  No profiling events are recorded.
 * The QK-norm + rotary prologue is not available here (its keys need a
 * workspace): a call with one is refused with LTXATTN_ERR_UNSUPPORTED.
 * The first call on a device sets it up (CU count, kernel attributes, the
 * scratch's device address); later calls only plan and launch.
 * Errors: INVALID_ARG, UNSUPPORTED (as ltxattn_block_attention), SCRATCH
 * (all before any launch), HIP (see ltxattn_last_hip_error(NULL)). */
int ltxattn_block_attention_noalloc(const ltxattn_config *cfg, const ltxattn_block_io *io, void *hip_stream);

/* Validate a block call against a configuration without touching any
 * device: returns the status ltxattn_block_attention would return from its
 * checks on a 256-CU MI355X (LTXATTN_OK if the call would be launched): the
 * arguments, then the workspace each kind's split parts need against the
 * handle's regions.  Lets a caller check a request up front, and the checks
 * be tested on a machine without a GPU. */
int ltxattn_check_block(const ltxattn_config *cfg, const ltxattn_block_io *io);

/* Free the workspace and the handle.  The caller must make sure no work
 * enqueued with the handle is still running.  NULL is accepted. */
int ltxattn_destroy(ltxattn_handle *h);

/* Static description of a status code. */
const char *ltxattn_status_string(int status);

/* The hipError_t behind the last LTXATTN_ERR_HIP (or OOM) returned for
 * this handle; with h == NULL, that of the last failed ltxattn_create or
 * ltxattn_block_attention_noalloc on the calling thread.  0 if none. */
int ltxattn_last_hip_error(const ltxattn_handle *h);

/* Per-kind timing with HIP events recorded on the stream each kind runs on.
 * ltxattn_profile_begin creates events for up to max_calls block calls
 * (created here, outside any timed region); each later block call (either
 * entry point) records an event where the call starts, where each kind ends
 * (a kind that follows another on the same stream starts at that event),
 * one after each kind's attention kernel when a combine kernel follows, and,
 * for the overlap entry point, where the audio side starts and where the
 * call ends after the join: 7 events per sequential call at the headline
 * shapes, each recorded between kernels that run back to back anyway.
 * ltxattn_profile_read waits for the recorded events and writes
 * LTXATTN_PROFILE_FLOATS floats per recorded call c < *n_calls (at most
 * max_calls), in milliseconds:
 *   ms[c*9 + kind]      that kind, all its kernels (0 if skipped);
 *   ms[c*9 + 4]         the whole call;
 *   ms[c*9 + 5 + kind]  that kind's attention kernel alone, without the
 *                       combine kernel that merges key-range parts.
 * ltxattn_profile_end stops recording and frees the events.
 * ltxattn_profile_begin_kinds records only the kinds whose bit (1 << kind)
 * is set in kind_mask (1..15), so that a timed loop carries only the events
 * it needs (each costs a few microseconds of device time): 3 per call for
 * VIDEO_SELF alone at the headline shapes.  Kinds outside the mask, and the
 * whole-call figure unless kind_mask is 15, read as NaN.
 * ltxattn_profile_begin(h, n) is ltxattn_profile_begin_kinds(h, n, 15).
 * Errors: INVALID_ARG (null pointer, max_calls < 1, kind_mask out of
 * range), HIP. */
#define LTXATTN_PROFILE_FLOATS 9
int ltxattn_profile_begin(ltxattn_handle *h, int32_t max_calls);
int ltxattn_profile_begin_kinds(ltxattn_handle *h, int32_t max_calls, uint32_t kind_mask);
int ltxattn_profile_read(ltxattn_handle *h, float *ms, int32_t max_calls, int32_t *n_calls);
int ltxattn_profile_end(ltxattn_handle *h);

#ifdef __cplusplus
}
#endif

#endif /* LTXATTN_H */

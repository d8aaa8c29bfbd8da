// ltxattn.hip -- the per-block attention set of the LTX-2 joint video+audio
// DiT on MI355X (gfx950): hand-written flash-attention kernels on bf16 MFMA
// and the C ABI declared in include/ltxattn.h.
//
// The four attentions (video self, audio self, a2v = video Q x audio KV,
// v2a = audio Q x video KV) are named in TensorRT-LLM PR #16228 "LTX-2:
// replicate audio stream across Ulysses ranks by default", "Description".
// Each computes O = softmax(Q K^T / sqrt(D)) V with bf16 inputs, fp32
// accumulation and fp32 softmax statistics.
//
// Kernel design (gfx950, 64-wide waves):
//  * Each wave owns 32 query rows of one (batch, head); keys stream through
//    in tiles of BN = 64.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K is the A operand (from LDS) and Q^T the B
//    operand (held in registers for the whole kernel).  In the 32x32
//    accumulator a lane then holds ONE query (lane % 32) and 16 keys, so
//    the online-softmax row max/sum is a per-lane loop plus one exchange
//    between the two half-waves (v_permlane32_swap).
//  * The output is accumulated transposed as well, O^T += V^T P^T: the
//    probabilities P^T are the B operand straight from the score
//    accumulators (converted to bf16 in registers, no LDS round trip) and
//    V^T is the A operand, read from the row-major V tile in LDS with the
//    transposing ds_read_b64_tr_b16.  Because a reduction index may be
//    permuted freely, the key order the score accumulator happens to give
//    each half-wave is simply used for V as well.
//  * K and V tiles go HBM -> LDS with buffer_load ... lds (no VGPR
//    staging).  Buffer range checks return zeros for rows past the valid
//    length, which handles ragged tails and the audio key padding without
//    branches; the padded keys are never read.  LDS rows are XOR-swizzled
//    per tensor so the K reads (16 rows per pass) and the transposed V
//    reads (4 rows per pass) are free of bank conflicts.
//  * Workgroups are remapped so that each of the 8 XCDs works through a
//    contiguous range of items and the K/V of a head stay in its L2.
//  * Items can be split over the key range: each part writes an
//    unnormalised fp32 partial O plus its row max and row sum, and a
//    combine kernel merges the parts by log-sum-exp in a fixed order (the
//    softmax statistics merge that the context-parallel v2a of
//    TensorRT-Model-Connect PR #1586 does across ranks).
//  * Kernels per kind (one block call launches them in this order):
//      video self   fa_ring_kernel<D, 8, 1>: 256-query items, one 8-wave
//                   workgroup per CU, a 4-stage K/V ring in LDS with
//                   partial load waits, loaded by the four waves that run
//                   behind their SIMD partners; each step is the score
//                   MFMAs of tile t+1, the probabilities of tile t (against
//                   the max in use, checked by their row sums) and its P V
//                   MFMAs.  The items of an incomplete last round run as
//                   key-range halves so the round fills its XCD; when they
//                   fill half of it, the first halves are dealt first and
//                   the second halves last, which keeps the two halves of
//                   the CUs changing items half an item apart.
//      v2a          fa_ring_kernel<D, 8, 2>: every 128-query item (all the
//                   audio queries of a head) split over the video keys, one
//                   part per CU; two 4-wave groups take the two key halves
//                   of each tile (a wave reads all of its V operands before
//                   the step's refill) and merge in LDS; then
//                   fa_combine_kernel.
//      a2v, audio   fa_kvres_kernel: the few hundred audio keys of a head
//      self         stay in LDS while the query tiles stream past; Q and O
//                   move as whole rows through per-wave LDS slots (or Q
//                   straight into registers when the keys fill the LDS).
//      other shapes fa_fwd_kernel<D, 4> (two-buffer pipeline, 128-query
//                   items) for long key streams that the cases above do
//                   not cover, e.g. D = 64 or short video.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "ltxattn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int BN = 64;           // keys per tile
constexpr int BM_MAX = 256;      // most query rows per workgroup (8 waves x 32)
constexpr int WAVES_PER_CU = 8;  // 2 per SIMD: the register budget of the attention kernel
constexpr int NSPLIT_MAX = 16;   // key-range parts of a split work item
constexpr int RSRC_FLAGS = 0x00020000;  // raw buffer, 32-bit data format
constexpr int PROF_EVENTS = 14;         // per profiled block call, at most: start, end, 3 per kind

// QK-norm + rotary prologue of the queries of one attention (w == null:
// none): RMS norm of each (token, head) row over its D channels with the
// per-channel weight w, then rotation of channel pairs -- (i, i + D/2), or
// (2i, 2i + 1) when interleaved -- by the angle whose cosine and sine the
// tables hold for pair i at the row's token.  Computed in fp32 and rounded
// to bf16 where the queries are loaded.
struct QkPrologue {
    const float *w;           // [D]
    const float *cos, *sin;   // [rows][D/2]
    float eps;
    int interleaved;
};

struct FaArgs {
    const __bf16 *q, *k, *v;
    QkPrologue qp;    // of q
    int64_t q_sb, q_ss, q_sh;
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    __bf16 *o;
    int64_t o_sb, o_ss, o_sh;
    const __bf16 *g;  // output gate (null: none), o's shape
    int64_t g_sb, g_ss, g_sh;
    float *part_o;    // split items: [split index][part][bm][D] fp32, unnormalised
    float *part_ml;   // split items: [split index][part][bm][2] = (row max * log2e/sqrt(D), row sum)
    int B, H, Sq, kv_len;
    int n_qtiles;     // query tiles per (batch, head); item = bh * n_qtiles + qtile
    // Work is dealt in G groups (G = 8, one per XCD, or 1).  Group g owns items
    // [g * ipg, (g + 1) * ipg): the first wpg run whole, one workgroup each;
    // the remaining ipg - wpg run as nsplit parts of split_len keys.
    int groups, ipg, wpg;
    int nsplit, split_len;
    // Ring kernel, two parts per split item and as many split items per group
    // as half its CUs: part 0 of each split item is dealt first and part 1
    // last, the whole items in between (see fa_ring_kernel).
    int stagger;
    float scale_log2;  // log2(e) / sqrt(D)
    int total;         // workgroups in the grid
};

struct CombineArgs {
    const float *part_o, *part_ml;
    __bf16 *o;
    int64_t o_sb, o_ss, o_sh;
    const __bf16 *g;
    int64_t g_sb, g_ss, g_sh;
    int H, Sq, bm, n_qtiles, ipg, wpg, n_split_items, nsplit;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, RSRC_FLAGS);
}

// Swizzled 16-byte chunk of row r in an LDS tile with D bf16 per row.
// K tiles are read 16 rows at a time at one logical chunk (ds_read_b128):
// rotating the chunk by the row spreads those rows over all banks.  V tiles
// are read 4 rows x 4 chunks at a time (ds_read_b64_tr_b16): each row gets
// its own group of 4 chunks.
template <int D> __device__ __forceinline__ int swz_k(int r, int c) {
    constexpr int NCH = D / 8, RPB = 128 / D;
    return c ^ ((r / RPB) % NCH);
}
template <int D> __device__ __forceinline__ int swz_v(int r, int c) {
    constexpr int NCH = D / 8, RPB = 128 / D;
    return c ^ ((4 * (r / RPB)) % NCH);
}

// Per-lane byte offsets that do not change from tile to tile.
template <int D, int NW>
struct LaneOffsets {
    static constexpr int KS = D / 16, NDB = D / 32;
    static constexpr int PER_THREAD = BN * (D / 8) / (64 * NW);   // DMA chunks per thread per tile
    int k_rd[KS];          // K tile, ds_read_b128 for k-step s (key block 0; block 1 is +32 rows)
    int v_rd[NDB];         // V tile, ds_read_b64_tr_b16 for d block db (k-step s adds 16s rows)
    int k_src[PER_THREAD]; // global byte offset (minus the tile's first row) of each K chunk
    int v_src[PER_THREAD];
};

// Copy BN rows x D of one (batch, head) slice, starting at key row t0, from
// HBM into an LDS tile with buffer_load ... lds.  Each wave instruction
// fills 1 KB of LDS contiguously (lane i -> +16*i); the swizzle is applied by
// choosing which global chunk each lane fetches (src).  Rows past the
// resource's range read as zeros.
template <int D, int NW>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rsrc, const int *src, int soff,
                                         LDS_AS char *tile, int wave) {
#pragma unroll
    for (int n = 0; n < LaneOffsets<D, NW>::PER_THREAD; ++n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(tile + (n * NW + wave) * 1024), 16,
                                                 src[n], soff, 0, 0);
}

__device__ __forceinline__ float xhalf_max(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *(const f32x4 *)p; }

// The prologue on one query row held as MFMA B-operand fragments: qf[k] is
// channels 8(2k + hw) .. +7 of this lane's row (the lane of the other
// half-wave holds the other chunks), so the row's sum of squares takes one
// exchange between the half-waves, and both channels of every pair are in
// the same lane -- chunk k pairs with chunk k + KS/2 (channel + D/2), or a
// pair is two neighbours within a chunk.  In two steps, so that a kernel
// can issue the loads of the weights and of the row's table entries early
// and apply them once its queries have arrived: q_prologue_load fills the
// lane's D/4 float4 of weights and table entries for table row `row`,
// q_prologue_apply normalises, rotates and rounds qf in place.
template <int D>
__device__ __forceinline__ void q_prologue_load(const QkPrologue &p, int row, int hw, f32x4 *t) {
    constexpr int KS = D / 16, P = D / 2;
    const float *cs = p.cos + (int64_t)row * P, *sn = p.sin + (int64_t)row * P;
    if (!p.interleaved) {
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) {
            const int d0 = 8 * (2 * k + hw);   // channels d0 .. d0+7 pair with d0+P ..
            t[8 * k + 0] = ld4(p.w + d0);
            t[8 * k + 1] = ld4(p.w + d0 + 4);
            t[8 * k + 2] = ld4(p.w + d0 + P);
            t[8 * k + 3] = ld4(p.w + d0 + P + 4);
            t[8 * k + 4] = ld4(cs + d0);
            t[8 * k + 5] = ld4(cs + d0 + 4);
            t[8 * k + 6] = ld4(sn + d0);
            t[8 * k + 7] = ld4(sn + d0 + 4);
        }
    } else {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int c8 = 8 * (2 * k + hw);   // channels c8 .. c8+7 = pairs c8/2 .. c8/2+3
            t[4 * k + 0] = ld4(p.w + c8);
            t[4 * k + 1] = ld4(p.w + c8 + 4);
            t[4 * k + 2] = ld4(cs + c8 / 2);
            t[4 * k + 3] = ld4(sn + c8 / 2);
        }
    }
}

template <int D>
__device__ __forceinline__ void q_prologue_apply(const QkPrologue &p, bf16x8 *qf, const f32x4 *t) {
    constexpr int KS = D / 16;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf((float)qf[k][j], (float)qf[k][j], ss);
    const float r = rsqrtf(fmaf(xhalf_sum(ss), 1.0f / D, p.eps));
    if (!p.interleaved) {
#pragma unroll
        for (int k = 0; k < KS / 2; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int h = j / 4, e = j % 4;
                const float ya = (float)qf[k][j] * r * t[8 * k + h][e];
                const float yc = (float)qf[k + KS / 2][j] * r * t[8 * k + 2 + h][e];
                const float cj = t[8 * k + 4 + h][e], sj = t[8 * k + 6 + h][e];
                qf[k][j] = (__bf16)(ya * cj - yc * sj);
                qf[k + KS / 2][j] = (__bf16)(ya * sj + yc * cj);
            }
    } else {
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ya = (float)qf[k][2 * j] * r * t[4 * k + j / 2][(2 * j) % 4];
                const float yc = (float)qf[k][2 * j + 1] * r * t[4 * k + j / 2][(2 * j + 1) % 4];
                const float cj = t[4 * k + 2][j], sj = t[4 * k + 3][j];
                qf[k][2 * j] = (__bf16)(ya * cj - yc * sj);
                qf[k][2 * j + 1] = (__bf16)(ya * sj + yc * cj);
            }
    }
}

// The prologue in one step, a quarter of the weights and table entries at a
// time (scheduling barriers keep the compiler from loading them all at
// once), for kernels whose registers are mostly taken.
template <int D>
__device__ __forceinline__ void q_prologue(const QkPrologue &p, bf16x8 *qf, int row, int hw) {
    constexpr int KS = D / 16, P = D / 2;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf((float)qf[k][j], (float)qf[k][j], ss);
    const float r = rsqrtf(fmaf(xhalf_sum(ss), 1.0f / D, p.eps));
    const float *cs = p.cos + (int64_t)row * P, *sn = p.sin + (int64_t)row * P;
    if (!p.interleaved) {
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) {
            const int d0 = 8 * (2 * k + hw);
            const f32x4 wa[2] = {ld4(p.w + d0), ld4(p.w + d0 + 4)}, wc[2] = {ld4(p.w + d0 + P), ld4(p.w + d0 + P + 4)};
            const f32x4 c[2] = {ld4(cs + d0), ld4(cs + d0 + 4)}, sv[2] = {ld4(sn + d0), ld4(sn + d0 + 4)};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float ya = (float)qf[k][j] * r * wa[j / 4][j % 4];
                const float yc = (float)qf[k + KS / 2][j] * r * wc[j / 4][j % 4];
                const float cj = c[j / 4][j % 4], sj = sv[j / 4][j % 4];
                qf[k][j] = (__bf16)(ya * cj - yc * sj);
                qf[k + KS / 2][j] = (__bf16)(ya * sj + yc * cj);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int c8 = 8 * (2 * k + hw);
            const f32x4 w[2] = {ld4(p.w + c8), ld4(p.w + c8 + 4)};
            const f32x4 c = ld4(cs + c8 / 2), sv = ld4(sn + c8 / 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ya = (float)qf[k][2 * j] * r * w[j / 2][(2 * j) % 4];
                const float yc = (float)qf[k][2 * j + 1] * r * w[j / 2][(2 * j + 1) % 4];
                qf[k][2 * j] = (__bf16)(ya * c[j] - yc * sv[j]);
                qf[k][2 * j + 1] = (__bf16)(ya * sv[j] + yc * c[j]);
            }
            if (k % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The prologue as a pass of its own, for keys (which reach LDS by DMA, with
// no register stage to fuse it into): y = prologue(x), [B][S][H][D] bf16
// contiguous.  One wave per token: a lane holds 8 consecutive channels
// (16-byte loads and stores) of one head, D/8 lanes a head and 64/(D/8)
// heads at a time, so the lane's table entries -- the same for every head of
// the token -- are loaded once.  Rotate-half partners sit D/16 lanes apart
// and trade values by one exchange.
struct PrologueRowsArgs {
    const __bf16 *x;
    int64_t x_sb, x_ss, x_sh;
    __bf16 *y;
    QkPrologue p;
    int S, H;
    int64_t tokens;   // B * S
};

constexpr int PASS_UNROLL = 4;   // head groups whose loads are issued together

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void qk_prologue_kernel(const PrologueRowsArgs a) {
    constexpr int LPR = D / 8, HPW = 64 / LPR, P = D / 2;   // lanes per head, heads per wave
    const int lane = threadIdx.x & 63, c = lane % LPR, hr = lane / LPR, d0 = 8 * c;
    const bool lower = d0 < P;                              // rotate-half: holds the first channel of its pairs
    const int i0 = a.p.interleaved ? d0 / 2 : d0 % P;       // first pair index of the lane's channels
    const f32x4 w0 = ld4(a.p.w + d0), w1 = ld4(a.p.w + d0 + 4);
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); tok < a.tokens; tok += nwaves) {
        const int s = (int)(tok % a.S);
        const int64_t b = tok / a.S;
        const float *ct = a.p.cos + (int64_t)s * P + i0, *st = a.p.sin + (int64_t)s * P + i0;
        const f32x4 cs[2] = {ld4(ct), a.p.interleaved ? f32x4{} : ld4(ct + 4)};
        const f32x4 sn[2] = {ld4(st), a.p.interleaved ? f32x4{} : ld4(st + 4)};
        const __bf16 *xt = a.x + b * a.x_sb + (int64_t)s * a.x_ss + d0;
        __bf16 *yt = a.y + tok * a.H * D + d0;
        for (int h0 = 0; h0 < a.H; h0 += HPW * PASS_UNROLL) {
            bf16x8 xv[PASS_UNROLL];
#pragma unroll
            for (int u = 0; u < PASS_UNROLL; ++u) {
                const int h = min(h0 + u * HPW + hr, a.H - 1);
                xv[u] = *(const bf16x8 *)(xt + (int64_t)h * a.x_sh);
            }
#pragma unroll
            for (int u = 0; u < PASS_UNROLL; ++u) {
                const int h = h0 + u * HPW + hr;
                float y[8], ss = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    y[j] = (float)xv[u][j];
                    ss = fmaf(y[j], y[j], ss);
                }
#pragma unroll
                for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
                const float r = rsqrtf(fmaf(ss, 1.0f / D, a.p.eps));
#pragma unroll
                for (int j = 0; j < 8; ++j) y[j] = y[j] * r * (j < 4 ? w0[j] : w1[j - 4]);
                bf16x8 out;
                if (a.p.interleaved) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float cj = cs[0][j], sj = sn[0][j];
                        out[2 * j] = (__bf16)(y[2 * j] * cj - y[2 * j + 1] * sj);
                        out[2 * j + 1] = (__bf16)(y[2 * j] * sj + y[2 * j + 1] * cj);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float other = __shfl_xor(y[j], LPR / 2, 64);   // the partner channel, D/2 away
                        const float cj = cs[j / 4][j % 4], sj = sn[j / 4][j % 4];
                        out[j] = (__bf16)(lower ? y[j] * cj - other * sj : other * sj + y[j] * cj);
                    }
                }
                if (h < a.H) *(bf16x8 *)(yt + (int64_t)h * D) = out;
            }
        }
    }
}

// Wait for all of this wave's outstanding memory loads (including DMA into
// LDS), then synchronise the workgroup.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// Rescaling of the running output is skipped until some row's max has grown
// by more than 2^RESCALE_LOG2 over the max in use: until then probabilities
// are taken against the stale max and stay below 2^RESCALE_LOG2.  Exact
// algebra: O / l does not depend on which max was subtracted.
constexpr float RESCALE_LOG2 = 8.0f;
// The same bound on a lane's sum of probabilities in one tile: a sum at most
// 2^RESCALE_LOG2 has every term at most 2^RESCALE_LOG2.
constexpr float RESCALE_SUM = 256.0f;

// One output row from its O^T fragments (o[db][i*4+j] = O^T[32db + 8i + 4hw + j]):
// bf16(acc * inv), or bf16((acc * inv) * gate) with a gate row.
template <int NDB>
__device__ __forceinline__ void store_row(__bf16 *orow, const __bf16 *grow, bool gated, const f32x16 *o,
                                          float inv, int hw) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = 32 * db + 8 * i + 4 * hw;
            bf16x4 ov;
            if (gated) {
                const bf16x4 gv = *(const bf16x4 *)(grow + col);
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = (__bf16)((o[db][i * 4 + j] * inv) * (float)gv[j]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(o[db][i * 4 + j] * inv);
            }
            *(bf16x4 *)(orow + col) = ov;
        }
}

template <int D>
struct RowState {
    f32x16 o[D / 32];   // O^T accumulator: o[db][i*4+j] = O^T[32db + 8i + 4hw + j][query]
    float m;            // max in use (raw score units)
    float l;            // this half-wave's share of the row sum
};

struct TileCtx {
    __amdgpu_buffer_rsrc_t kr, vr;
    int k_stride, v_stride;   // bytes per key row
    int kv_end;
    float c;                  // log2(e) / sqrt(D)
    int wave, hw;
};

// The softmax and MFMA helpers below take NK keys per call: the whole tile
// (BN), or 32 when a tile's keys are shared out between two wave groups.

// S^T = K Q^T for one tile: s[kb][i*4+j] is the score of key t0 + 32kb + 8i +
// 4hw + j against this lane's query.
template <int D, int NW, int NK = BN>
__device__ __forceinline__ void scores(const LaneOffsets<D, NW> &lo, const bf16x8 *qf,
                                       const LDS_AS char *__restrict__ ktile, f32x16 *s) {
    constexpr int KS = D / 16, NKB = NK / 32;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    // k outer, key block inner: the NKB accumulator chains are independent,
    // so consecutive MFMAs do not wait on each other's results.
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const u32x4 w = *(const LDS_AS u32x4 *)(ktile + kb * 32 * 2 * D + lo.k_rd[k]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), qf[k], s[kb], 0, 0, 0);
        }
    }
}

// Keys at or past kv_end (ragged tail, audio padding) get -inf.
template <int NK = BN>
__device__ __forceinline__ void mask_tail(const TileCtx &x, int t0, f32x16 *s) {
    constexpr int NKB = NK / 32;
    if (t0 + NK > x.kv_end) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = t0 + 32 * kb + 8 * (e >> 2) + 4 * x.hw + (e & 3);
                if (key >= x.kv_end) s[kb][e] = -INFINITY;
            }
    }
}

// Online softmax, first half: the tile's row max, and a lazy update of the
// max in use -- O and the row sum are rescaled only if some row's max grew
// by more than 2^RESCALE_LOG2.
template <int D, int NK = BN>
__device__ __forceinline__ void update_max(const TileCtx &x, const f32x16 *s, RowState<D> &st) {
    constexpr int NDB = D / 32, NKB = NK / 32;
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            mx0 = fmaxf(fmaxf(mx0, s[kb][e]), s[kb][e + 1]);        // v_max3
            mx1 = fmaxf(fmaxf(mx1, s[kb][e + 2]), s[kb][e + 3]);
        }
    const float mx = xhalf_max(fmaxf(mx0, mx1));
    if (__builtin_amdgcn_ballot_w64((mx - st.m) * x.c > RESCALE_LOG2)) {
        const float m_new = fmaxf(st.m, mx);
        const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * x.c);
        st.m = m_new;
        st.l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[db][e] *= alpha;
    }
}

// Online softmax, second half: P = 2^(S c - m c) in bf16, packed in MFMA
// B-operand order -- k-step k of the PV product takes keys 16k + 4hw +
// {0..3} and 16k + 8 + 4hw + {0..3}, i.e. accumulator rows i = 2(k%2) and
// 2(k%2)+1 of block k/2 -- and the row sum of exactly these bf16 weights
// (v_dot2 with ones).
template <int D, int NK = BN>
__device__ __forceinline__ void probs(const TileCtx &x, const f32x16 *s, RowState<D> &st, bf16x8 *pf) {
    constexpr int PS = NK / 16;
    const float mc = st.m * x.c;
    float rs0 = 0.f, rs1 = 0.f;
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int k = 0; k < PS; ++k) {
        const int kb = k >> 1, i0 = 2 * (k & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pf[k][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][i0 * 4 + j], x.c, -mc));
            pf[k][4 + j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][(i0 + 1) * 4 + j], x.c, -mc));
        }
#pragma unroll
        for (int j = 0; j < 8; j += 4) {
            rs0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[k][j], pf[k][j + 1]}, one, rs0, false);
            rs1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[k][j + 2], pf[k][j + 3]}, one, rs1, false);
        }
    }
    st.l += rs0 + rs1;
}

// O^T += V^T P^T for one tile.  V^T comes from the row-major V tile via the
// transposing read: 16 lanes read 4 key rows x 16 d, each lane ending up
// with 4 keys of one d column.
template <int D, int NW, int NK = BN>
__device__ __forceinline__ void accumulate_pv(const LaneOffsets<D, NW> &lo, const LDS_AS char *__restrict__ vtile,
                                              const bf16x8 *pf, RowState<D> &st) {
    constexpr int NDB = D / 32, PS = NK / 16;
#pragma unroll
    for (int k = 0; k < PS; ++k) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const LDS_AS char *vp = vtile + lo.v_rd[db] + k * 16 * 2 * D;
            const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)vp);
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vp + 8 * 2 * D));
            const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[k], st.o[db], 0, 0, 0);
        }
    }
}

// One pipelined step, for tile t whose scores s_cur are already computed.
// K runs one tile ahead of V: this step prefetches K of tile t+2 and V of
// tile t+1, settles the max of tile t, then -- in one straight-line block
// the scheduler can interleave -- computes the scores of tile t+1 (MFMA)
// while the probabilities of tile t are formed (VALU), and accumulates
// P V of tile t.  The scores of t+1 are computed even past the last tile
// (from a stale buffer, in bounds) and then simply not used.  Each tensor
// has two LDS buffers; the tiles are restrict pointers, so the compiler
// knows the reads do not touch the buffers being refilled.
template <int D, int NW>
__device__ __forceinline__ void pipeline_step(const TileCtx &x, const LaneOffsets<D, NW> &lo, const bf16x8 *qf,
                                              RowState<D> &st, const f32x16 *s_cur, f32x16 *s_next,
                                              int t0, int ntiles_left,
                                              const LDS_AS char *__restrict__ k_next,   // K of t+1
                                              const LDS_AS char *__restrict__ v_cur,    // V of t
                                              LDS_AS char *__restrict__ k_fill,         // <- K of t+2
                                              LDS_AS char *__restrict__ v_fill) {       // <- V of t+1
    constexpr int PS = BN / 16;
    if (ntiles_left > 2) dma_tile<D, NW>(x.kr, lo.k_src, (t0 + 2 * BN) * x.k_stride, k_fill, x.wave);
    if (ntiles_left > 1) dma_tile<D, NW>(x.vr, lo.v_src, (t0 + BN) * x.v_stride, v_fill, x.wave);
    update_max<D>(x, s_cur, st);
    bf16x8 pf[PS];
    scores<D, NW>(lo, qf, k_next, s_next);
    probs<D>(x, s_cur, st, pf);
    accumulate_pv<D, NW>(lo, v_cur, pf, st);
    mask_tail(x, t0 + BN, s_next);
}

template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2)))
void fa_fwd_kernel(const FaArgs a) {
    constexpr int BM = 32 * NW;        // query rows per workgroup
    constexpr int KS = D / 16, NDB = D / 32, NCH = D / 8, NKB = BN / 32;
    constexpr int TILE = BN * D * 2;   // bytes of one K or V tile
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K0 K1 V0 V1
    LDS_AS char *const lds = (LDS_AS char *)smem;
    LDS_AS char *const K0 = lds, *const K1 = lds + TILE, *const V0 = lds + 2 * TILE, *const V1 = lds + 3 * TILE;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = lane >> 5, l32 = lane & 31;

    // Blocks are dealt to the 8 XCDs round-robin, so with 8 groups block
    // bid runs on XCD bid % 8 and group g = bid % 8 keeps one contiguous
    // range of items (same heads -> shared K/V) in that XCD's L2.  Within a
    // group: whole items first (query tile fastest), then the parts of the
    // split items.
    const int bid = blockIdx.x;
    const int g = bid % a.groups, local = bid / a.groups;
    const bool split_item = local >= a.wpg;
    const int w = local - a.wpg;
    const int part = split_item ? w % a.nsplit : 0;
    const int item = g * a.ipg + (split_item ? a.wpg + w / a.nsplit : local);
    const int split_idx = g * (a.ipg - a.wpg) + (split_item ? w / a.nsplit : 0);
    const int qt = item % a.n_qtiles;
    const int bh = item / a.n_qtiles;
    const int b = bh / a.H, hh = bh % a.H;
    const int kv_begin = part * a.split_len;

    TileCtx x;
    x.kv_end = split_item ? min(a.kv_len, kv_begin + a.split_len) : a.kv_len;
    x.c = a.scale_log2;
    x.wave = wave;
    x.hw = hw;
    x.k_stride = (int)(a.k_ss * 2);
    x.v_stride = (int)(a.v_ss * 2);
    const __bf16 *qb = a.q + b * a.q_sb + hh * a.q_sh;
    x.kr = make_rsrc(a.k + b * a.k_sb + hh * a.k_sh, ((int64_t)(a.kv_len - 1) * a.k_ss + D) * 2);
    x.vr = make_rsrc(a.v + b * a.v_sb + hh * a.v_sh, ((int64_t)(a.kv_len - 1) * a.v_ss + D) * 2);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qb, ((int64_t)(a.Sq - 1) * a.q_ss + D) * 2);

    LaneOffsets<D, NW> lo;
#pragma unroll
    for (int n = 0; n < LaneOffsets<D, NW>::PER_THREAD; ++n) {
        const int idx = (n * NW + wave) * 64 + lane;   // physical chunk index in the tile
        const int r = idx / NCH, p = idx % NCH;
        lo.k_src[n] = r * x.k_stride + swz_k<D>(r, p) * 16;   // the swizzle is an involution
        lo.v_src[n] = r * x.v_stride + swz_v<D>(r, p) * 16;
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) lo.k_rd[k] = l32 * 2 * D + swz_k<D>(l32, 2 * k + hw) * 16;
    {
        const int li = lane & 15, g = (lane >> 4) & 1;
        const int r0 = 4 * hw + (li >> 2);   // + 16k (+8) added as immediates
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * g + 4 * (li & 3);
            lo.v_rd[db] = r0 * 2 * D + swz_v<D>(r0, col >> 3) * 16 + ((col >> 2) & 1) * 8;
        }
    }

    const int ntiles = (x.kv_end - kv_begin + BN - 1) / BN;
    dma_tile<D, NW>(x.kr, lo.k_src, kv_begin * x.k_stride, K0, wave);
    dma_tile<D, NW>(x.vr, lo.v_src, kv_begin * x.v_stride, V0, wave);
    if (ntiles > 1) dma_tile<D, NW>(x.kr, lo.k_src, (kv_begin + BN) * x.k_stride, K1, wave);

    // Q^T as the B operand: lane holds 8 consecutive d of its query row per k-step.
    const int qrow = qt * BM + wave * 32 + l32;
    bf16x8 qf[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            qr, (int)((int64_t)qrow * a.q_ss * 2) + (2 * k + hw) * 16, 0, 0));
        qf[k] = __builtin_bit_cast(bf16x8, w);
    }
    if (a.qp.w) q_prologue<D>(a.qp, qf, min(qrow, a.Sq - 1), hw);

    RowState<D> st;
#pragma unroll
    for (int i = 0; i < NDB; ++i) st.o[i] = f32x16{};
    st.m = -1e30f;   // finite start: no inf - inf
    st.l = 0.f;

    // Before each barrier this wave waits for its own outstanding loads --
    // the DMA issued one step earlier (and, first time round, Q) -- so after
    // the barrier those tiles are in LDS and every wave is done with the
    // buffers the next prefetch refills.  The wait is explicit: the
    // compiler's own accounting does not cover LDS written by DMA across the
    // loop back-edge.  Two steps per trip keep every buffer a compile-time
    // offset.
    f32x16 sA[NKB], sB[NKB];
    tile_barrier();
    scores<D, NW>(lo, qf, K0, sA);
    mask_tail(x, kv_begin, sA);
    int t = 0;
    for (; t + 2 <= ntiles; t += 2) {
        const int t0 = kv_begin + t * BN;
        tile_barrier();
        pipeline_step<D, NW>(x, lo, qf, st, sA, sB, t0, ntiles - t, K1, V0, K0, V1);
        tile_barrier();
        pipeline_step<D, NW>(x, lo, qf, st, sB, sA, t0 + BN, ntiles - t - 1, K0, V1, K1, V0);
    }
    if (t < ntiles) {
        tile_barrier();
        pipeline_step<D, NW>(x, lo, qf, st, sA, sB, kv_begin + t * BN, ntiles - t, K1, V0, K0, V1);
    }

    // st.o[db][i*4+j] is O^T[d = 32db + 8i + 4hw + j][query qrow] (unnormalised).
    const float l_tot = xhalf_sum(st.l);
    if (!split_item) {
        if (qrow < a.Sq)
            store_row<NDB>(a.o + b * a.o_sb + (int64_t)qrow * a.o_ss + hh * a.o_sh,
                           a.g + b * a.g_sb + (int64_t)qrow * a.g_ss + hh * a.g_sh, a.g != nullptr,
                           st.o, 1.0f / l_tot, hw);
    } else {
        const int64_t prow = ((int64_t)split_idx * a.nsplit + part) * BM + (qrow - qt * BM);
        float *po = a.part_o + prow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = st.o[db][i * 4 + j];
                *(f32x4 *)(po + 32 * db + 8 * i + 4 * hw) = ov;
            }
        if (hw == 0) {
            a.part_ml[prow * 2 + 0] = st.m * x.c;
            a.part_ml[prow * 2 + 1] = l_tot;
        }
    }
}


// ------------------------------------------------ ring-pipelined streaming
// fa_ring_kernel streams one key range of one item through a ring of
// RING_STAGES (K, V) tile pairs in LDS and waits only for the oldest tile it
// needs: two tiles stay in flight at all times, where fa_fwd_kernel's two
// buffers drain their loads at every step.  One workgroup of NW waves per
// CU (the ring takes 128 KB of LDS at D = 128).  KG = 1: every wave owns 32
// queries (video self-attention, 256-query items).  KG = 2: v2a, whose
// queries of one head (the audio tokens) fit in one 128-query item while
// its keys run to tens of thousands -- the waves form two groups that both
// take all 128 queries, group g the keys 32g..32g+31 of every tile (two
// waves per SIMD instead of one), and the two running softmax states are
// merged through LDS at the end.  Items, parts and the combine of split
// items follow fa_fwd_kernel.
constexpr int RING_STAGES = 4;
constexpr int RING_NW = 8;

// Wait until at most N of this wave's loads are outstanding, then meet the
// other waves.  LDS written by a wave's loads is in place once its count
// has dropped, so a plain s_barrier is all the other waves need; a fence
// (as in __syncthreads) would also wait for the loads still meant to be in
// flight.  The empty asm statements keep the compiler from moving memory
// accesses across.
template <int N>
__device__ __forceinline__ void ring_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The ring, from the first loads to the last P V.  The eight stage buffers
// are restrict parameters of this one function: the compiler then tells
// every pending load from every LDS read and waits only where a read needs
// a tile, which the explicit waits have already covered.  Each step, for
// tile t whose scores are computed: wait for tile t+1 (tile t+2 may still
// be in flight), refill the stage of tile t-1 with tile t+3 -- from a
// zero-sized resource past the key range, so that every step issues the
// same number of loads and the wait count stays exact -- then the scores
// of t+1, the probabilities of t and P V of t, on this wave's NK keys of
// each tile (starting koff bytes into it).  The last LW waves of the
// workgroup issue the tile loads (chunk offsets in ldo); the others issue
// none and so never wait for them.  The compiler waits for every load into
// LDS still in flight before a transposing LDS read (it cannot tell which
// bytes such a read touches), so a wave that issued the current step's
// refill waits for it at its first V read of the step; with LW = NW / 2 the
// loads come from the waves that run behind their SIMD partners and reach
// that read latest.
template <int D, int NW, int NK, int LW, class Pre>
__device__ __forceinline__ void ring_loop(const TileCtx &x, const LaneOffsets<D, NW> &lo,
                                          const LaneOffsets<D, LW> &ldo, const bf16x8 *qf,
                                          RowState<D> &st, int kv_begin, int ntiles, int koff, int key0,
                                          __amdgpu_buffer_rsrc_t none, Pre &&pre,
                                          LDS_AS char *__restrict__ K0, LDS_AS char *__restrict__ K1,
                                          LDS_AS char *__restrict__ K2, LDS_AS char *__restrict__ K3,
                                          LDS_AS char *__restrict__ V0, LDS_AS char *__restrict__ V1,
                                          LDS_AS char *__restrict__ V2, LDS_AS char *__restrict__ V3) {
    constexpr int NKB = NK / 32, PS = NK / 16;
    constexpr int PER_TILE = 2 * LaneOffsets<D, LW>::PER_THREAD;   // loads per loading wave per tile
    auto load = [&](int i, bool f, LDS_AS char *kd, LDS_AS char *vd) {
        if (x.wave >= NW - LW) {   // uniform
            dma_tile<D, LW>(f ? x.kr : none, ldo.k_src, (kv_begin + i * BN) * x.k_stride, kd, x.wave - (NW - LW));
            dma_tile<D, LW>(f ? x.vr : none, ldo.v_src, (kv_begin + i * BN) * x.v_stride, vd, x.wave - (NW - LW));
        }
    };
    // The step at D = 128 (NK = 64, or 32 per key group), in three blocks:
    // the score MFMAs of tile t+1; the probabilities of tile t and their row
    // sums; the P V MFMAs of tile t.  Operand reads run LA k-steps ahead of
    // their MFMAs and scheduling barriers hold that order.  Every wave starts
    // the step at the same barrier; the two waves of a SIMD drift apart
    // within it, so one's MFMA blocks cover part of the other's exponentials.
    // Probabilities are taken against the max in use without computing the
    // tile's max first: if no lane's sum of its 2^(s c - m c) exceeds
    // RESCALE_SUM, none of them does either, which is the bound the lazy
    // rescale keeps; otherwise (the first tiles, or a new max) the wave takes
    // the tile's max, rescales and computes the probabilities again.
    auto step_sw = [&](const f32x16 *s_cur, f32x16 *s_next, int t, const LDS_AS char *k_next,
                       const LDS_AS char *v_cur, LDS_AS char *k_fill, LDS_AS char *v_fill) {
        constexpr int KS = D / 16, NDB = D / 32;
        constexpr int LA = 2;
        ring_barrier<PER_TILE>();
        auto read_v = [&](int c, bf16x8 *op) {
            const int k = c >> 1, dbp = c & 1;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const LDS_AS char *vp = v_cur + koff + lo.v_rd[2 * dbp + j] + k * 16 * 2 * D;
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)vp);
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vp + 8 * 2 * D));
                op[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };
        // Two key groups (NK = 32): all of this tile's V operands fit in
        // registers, so they are read before the refill is issued and the
        // compiler's wait for loads into LDS before the next step's first
        // transposed read covers a refill issued a whole step earlier.
        constexpr bool PRE_V = NK < BN;
        bf16x8 vall[PRE_V ? 2 * PS : 1][2];
        if constexpr (PRE_V) {
#pragma unroll
            for (int c = 0; c < 2 * PS; ++c) read_v(c, vall[c]);
            __builtin_amdgcn_sched_barrier(0);
        }
        load(t + 3, t + 3 < ntiles, k_fill, v_fill);

        bf16x8 kop[LA + 1][NKB];
        auto read_k = [&](int k, bf16x8 *op) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                op[kb] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4 *)(k_next + koff + kb * 32 * 2 * D + lo.k_rd[k]));
        };
#pragma unroll
        for (int c = 0; c < LA; ++c) read_k(c, kop[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < KS; ++c) {
            if (c + LA < KS) read_k(c + LA, kop[(c + LA) % (LA + 1)]);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                s_next[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c % (LA + 1)][kb], qf[c],
                                                                     c == 0 ? f32x16{} : s_next[kb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        mask_tail<NK>(x, key0 + (t + 1) * BN, s_next);

        // pf[k][4h + j] = 2^(s c - m c) of score s_cur[k / 2][4 (2 (k % 2) + h) + j]
        // (the B-operand order of P V k-step k), row sums in two chains.
        bf16x8 pf[PS];
        auto probs_sum = [&]() {
            const float mc = st.m * x.c;
            const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int k = 0; k < PS; ++k)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kb = k >> 1, i = 2 * (k & 1) + h;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pf[k][4 * h + j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s_cur[kb][i * 4 + j], x.c, -mc));
                    rs0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[k][4 * h], pf[k][4 * h + 1]}, one, rs0, false);
                    rs1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[k][4 * h + 2], pf[k][4 * h + 3]}, one, rs1, false);
                }
            return rs0 + rs1;
        };
        float rsum = probs_sum();
        if (__builtin_amdgcn_ballot_w64(!(rsum <= RESCALE_SUM))) {
            float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; e += 4) {
                    mx0 = fmaxf(fmaxf(mx0, s_cur[kb][e]), s_cur[kb][e + 1]);
                    mx1 = fmaxf(fmaxf(mx1, s_cur[kb][e + 2]), s_cur[kb][e + 3]);
                }
            const float m_new = fmaxf(st.m, xhalf_max(fmaxf(mx0, mx1)));
            const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * x.c);
            st.m = m_new;
            st.l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) st.o[db][e] *= alpha;
            rsum = probs_sum();
        }
        st.l += rsum;

        bf16x8 vop[LA + 1][2];
        if constexpr (PRE_V) {
#pragma unroll
            for (int c = 0; c < 2 * PS; ++c) {
                const int k = c >> 1, dbp = c & 1;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    st.o[2 * dbp + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vall[c][j], pf[k], st.o[2 * dbp + j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int c = 0; c < LA; ++c) read_v(c, vop[c]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < 2 * PS; ++c) {
                if (c + LA < 2 * PS) read_v(c + LA, vop[(c + LA) % (LA + 1)]);
                const int k = c >> 1, dbp = c & 1;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    st.o[2 * dbp + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[c % (LA + 1)][j], pf[k], st.o[2 * dbp + j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    auto step = [&](const f32x16 *s_cur, f32x16 *s_next, int t, const LDS_AS char *k_next,
                    const LDS_AS char *v_cur, LDS_AS char *k_fill, LDS_AS char *v_fill) {
        if constexpr (D == 128) {
            step_sw(s_cur, s_next, t, k_next, v_cur, k_fill, v_fill);
        } else {
            ring_barrier<PER_TILE>();
            load(t + 3, t + 3 < ntiles, k_fill, v_fill);
            update_max<D, NK>(x, s_cur, st);
            bf16x8 pf[PS];
            scores<D, NW, NK>(lo, qf, k_next + koff, s_next);
            probs<D, NK>(x, s_cur, st, pf);
            accumulate_pv<D, NW, NK>(lo, v_cur + koff, pf, st);
            mask_tail<NK>(x, key0 + (t + 1) * BN, s_next);
        }
    };
    // Q was loaded before this: the loads complete in issue order, so for a
    // loading wave the count still outstanding names exactly what has landed
    // (the others have no tile loads; the compiler waits for their Q).
    load(0, 0 < ntiles, K0, V0);
    load(1, 1 < ntiles, K1, V1);
    load(2, 2 < ntiles, K2, V2);
    pre();                          // work on Q before the first wait for tiles
    ring_barrier<2 * PER_TILE>();   // Q and tile 0
    f32x16 sA[NKB], sB[NKB];
    scores<D, NW, NK>(lo, qf, K0 + koff, sA);
    mask_tail<NK>(x, key0, sA);
    if constexpr (D == 128) update_max<D, NK>(x, sA, st);   // steps expect it settled
    int t = 0;
    for (; t + 4 <= ntiles; t += 4) {
        step(sA, sB, t, K1, V0, K3, V3);
        step(sB, sA, t + 1, K2, V1, K0, V0);
        step(sA, sB, t + 2, K3, V2, K1, V1);
        step(sB, sA, t + 3, K0, V3, K2, V2);
    }
    // 0..3 tiles left; the scores of tile t are in sA.
    if (t < ntiles) step(sA, sB, t, K1, V0, K3, V3);
    if (t + 1 < ntiles) step(sB, sA, t + 1, K2, V1, K0, V0);
    if (t + 2 < ntiles) step(sA, sB, t + 2, K3, V2, K1, V1);
    // Every wave is done with the ring, and the loads of tiles past the end
    // have landed, before its LDS is reused or released.
    ring_barrier<0>();
}

template <int D, int NW, int KG, bool QP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2)))
void fa_ring_kernel(const FaArgs a) {
    constexpr int QW = NW / KG;                 // waves per key group = 32-query blocks per item
    constexpr int BM = 32 * QW, NK = BN / KG;
    constexpr int KS = D / 16, NDB = D / 32, NCH = D / 8;
    constexpr int TILE = BN * D * 2;
    // K stages 0..3, then V stages 0..3: each kind's reads then reach all
    // its stages by immediate offsets (< 64 KB) from one address per lane.
    extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];
    LDS_AS char *const lds = (LDS_AS char *)smem_dyn;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = wave / QW, wq = wave % QW;
    const int hw = lane >> 5, l32 = lane & 31;

    // Item decode: group g = XCD.  By default as in fa_fwd_kernel, whole
    // items first, then the parts of the split items.  Staggered: the first
    // spg workgroups of a group are part 0 of its split items, then the whole
    // items, then the part 1s.  Half of the XCD's CUs then start with a
    // half-length item and run half an item out of phase with the other half
    // until the part 1s even them out at the end, so the CUs do not all
    // change items (epilogue, Q load, first tiles) at the same moment.
    const int bid = blockIdx.x;
    const int g = bid % a.groups, local0 = bid / a.groups;
    const int spg = a.ipg - a.wpg;   // split items per group
    bool split_item;
    int local, part, sidx;           // whole item index, or part and split item index
    if (a.stagger) {
        split_item = local0 < spg || local0 >= spg + a.wpg;
        local = local0 - spg;
        part = local0 >= spg + a.wpg ? 1 : 0;
        sidx = local0 < spg ? local0 : local0 - spg - a.wpg;
    } else {
        split_item = local0 >= a.wpg;
        local = local0;
        part = split_item ? (local0 - a.wpg) % a.nsplit : 0;
        sidx = split_item ? (local0 - a.wpg) / a.nsplit : 0;
    }
    const int item = g * a.ipg + (split_item ? a.wpg + sidx : local);
    const int split_idx = g * spg + (split_item ? sidx : 0);
    const int qt = item % a.n_qtiles, bh = item / a.n_qtiles;
    const int b = bh / a.H, hh = bh % a.H;
    const int kv_begin = part * a.split_len;

    TileCtx x;
    x.kv_end = split_item ? min(a.kv_len, kv_begin + a.split_len) : a.kv_len;
    x.c = a.scale_log2;
    x.wave = wave;
    x.hw = hw;
    x.k_stride = (int)(a.k_ss * 2);
    x.v_stride = (int)(a.v_ss * 2);
    x.kr = make_rsrc(a.k + b * a.k_sb + hh * a.k_sh, ((int64_t)(a.kv_len - 1) * a.k_ss + D) * 2);
    x.vr = make_rsrc(a.v + b * a.v_sb + hh * a.v_sh, ((int64_t)(a.kv_len - 1) * a.v_ss + D) * 2);
    const __amdgpu_buffer_rsrc_t none = make_rsrc(a.k, 0);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + b * a.q_sb + hh * a.q_sh, ((int64_t)(a.Sq - 1) * a.q_ss + D) * 2);

    // Tile loads come from the last LW waves: half of them for video
    // self-attention, all of them when two key groups split each tile.
    constexpr int LW = KG == 1 ? NW / 2 : NW;
    const int lw = wave >= NW - LW ? wave - (NW - LW) : 0;
    LaneOffsets<D, LW> ldo;
#pragma unroll
    for (int n = 0; n < LaneOffsets<D, LW>::PER_THREAD; ++n) {
        const int idx = (n * LW + lw) * 64 + lane;
        const int r = idx / NCH, p = idx % NCH;
        ldo.k_src[n] = r * x.k_stride + swz_k<D>(r, p) * 16;
        ldo.v_src[n] = r * x.v_stride + swz_v<D>(r, p) * 16;
    }
    LaneOffsets<D, NW> lo;   // LDS read offsets
#pragma unroll
    for (int k = 0; k < KS; ++k) lo.k_rd[k] = l32 * 2 * D + swz_k<D>(l32, 2 * k + hw) * 16;
    {
        const int li = lane & 15, gg = (lane >> 4) & 1;
        const int r0 = 4 * hw + (li >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * gg + 4 * (li & 3);
            lo.v_rd[db] = r0 * 2 * D + swz_v<D>(r0, col >> 3) * 16 + ((col >> 2) & 1) * 8;
        }
    }

    const int qrow = qt * BM + wq * 32 + l32;
    bf16x8 qf[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k)
        qf[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
            qr, (int)((int64_t)qrow * a.q_ss * 2) + (2 * k + hw) * 16, 0, 0));
    f32x4 qtab[QP ? D / 4 : 1];
    if constexpr (QP) q_prologue_load<D>(a.qp, min(qrow, a.Sq - 1), hw, qtab);
    const int ntiles = (x.kv_end - kv_begin + BN - 1) / BN;
    asm volatile("" ::: "memory");   // Q's loads stay ahead of the tiles'

    RowState<D> st;
#pragma unroll
    for (int i = 0; i < NDB; ++i) st.o[i] = f32x16{};
    st.m = -1e30f;
    st.l = 0.f;
    // The query prologue runs while the ring's first tiles are on their way.
    auto pre = [&]() { if constexpr (QP) q_prologue_apply<D>(a.qp, qf, qtab); };
    ring_loop<D, NW, NK, LW>(x, lo, ldo, qf, st, kv_begin, ntiles, group * NK * 2 * D, kv_begin + group * NK, none,
                         pre, lds, lds + TILE, lds + 2 * TILE, lds + 3 * TILE,
                         lds + 4 * TILE, lds + 5 * TILE, lds + 6 * TILE, lds + 7 * TILE);

    float l_tot = xhalf_sum(st.l);
    if (KG == 2) {
        // Merge the key halves: group 1 leaves its state in LDS (lane-major,
        // so the partner wave of group 0 -- same queries, same lane layout --
        // reads exactly its own elements), group 0 folds it in.
        LDS_AS char *const mo = lds + wq * (NDB * 16 * 64 * 4);
        LDS_AS float *const mm = (LDS_AS float *)(lds + QW * NDB * 16 * 64 * 4) + wq * 128;
        if (group == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = st.o[db][i * 4 + j];
                    *(LDS_AS f32x4 *)(mo + ((db * 4 + i) * 64 + lane) * 16) = v;
                }
            mm[lane] = st.m;
            mm[64 + lane] = l_tot;
        }
        __syncthreads();
        if (group == 1) return;
        const float m1 = mm[lane], l1 = mm[64 + lane];
        const float m_new = fmaxf(st.m, m1);
        const float a0 = __builtin_amdgcn_exp2f((st.m - m_new) * x.c);
        const float a1 = __builtin_amdgcn_exp2f((m1 - m_new) * x.c);
        st.m = m_new;
        l_tot = a0 * l_tot + a1 * l1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v = *(const LDS_AS f32x4 *)(mo + ((db * 4 + i) * 64 + lane) * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j) st.o[db][i * 4 + j] = a0 * st.o[db][i * 4 + j] + a1 * v[j];
            }
    }

    // st.o[db][i*4+j] is O^T[d = 32db + 8i + 4hw + j][query qrow] (unnormalised).
    if (!split_item) {
        if (qrow < a.Sq)
            store_row<NDB>(a.o + b * a.o_sb + (int64_t)qrow * a.o_ss + hh * a.o_sh,
                           a.g + b * a.g_sb + (int64_t)qrow * a.g_ss + hh * a.g_sh, a.g != nullptr,
                           st.o, 1.0f / l_tot, hw);
    } else {
        const int64_t prow = ((int64_t)split_idx * a.nsplit + part) * BM + (qrow - qt * BM);
        float *po = a.part_o + prow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 ov;
#pragma unroll
                for (int j = 0; j < 4; ++j) ov[j] = st.o[db][i * 4 + j];
                *(f32x4 *)(po + 32 * db + 8 * i + 4 * hw) = ov;
            }
        if (hw == 0) {
            a.part_ml[prow * 2 + 0] = st.m * x.c;
            a.part_ml[prow * 2 + 1] = l_tot;
        }
    }
}

// ------------------------------------------------ resident short key streams
// One block of 32 queries (this wave's) against two key tiles held in LDS --
// at most 128 keys: K tiles at K and K + TILE, V tiles at V and V + TILE,
// rows past kv_end zero -- in one software-pipelined pass at D = 128: the
// score MFMAs of tile 1 run beside the probabilities of tile 0, and the P V
// MFMAs of tile 0 beside the probabilities of tile 1 (operand reads two
// chunks ahead, scheduling barriers holding the interleave).  Tile 0 sets
// the max; tile 1's probabilities are taken against it and checked with the
// row-sum bound of the ring kernel, which takes tile 1's max and rescales
// only when some lane's sum exceeds RESCALE_SUM.  st is overwritten.
template <int D, int NW>
__device__ __forceinline__ void kv2_block(const TileCtx &x, const LaneOffsets<D, NW> &lo, const bf16x8 *qf,
                                          const LDS_AS char *__restrict__ K, const LDS_AS char *__restrict__ V,
                                          RowState<D> &st) {
    static_assert(D == 128, "two-tile pass at D = 128");
    constexpr int KS = D / 16, NDB = D / 32, PS = BN / 16, TILE = BN * D * 2;
    constexpr int LA = 2;
    auto read_k = [&](const LDS_AS char *kt, int k, bf16x8 *op) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            op[kb] = __builtin_bit_cast(bf16x8, *(const LDS_AS u32x4 *)(kt + kb * 32 * 2 * D + lo.k_rd[k]));
    };
    // Chunk c of a tile's P V: k-step c / 2, d blocks 2 (c % 2) and 2 (c % 2) + 1.
    auto read_v = [&](const LDS_AS char *vt, int c, bf16x8 *op) {
        const int k = c >> 1, dbp = c & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const LDS_AS char *vp = vt + lo.v_rd[2 * dbp + j] + k * 16 * 2 * D;
            const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)vp);
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vp + 8 * 2 * D));
            op[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    // k-step kk of a tile's probabilities, in P V B-operand order (as in the
    // ring kernel), with its row sums.
    auto prob_step = [&](const f32x16 *sv, int kk, float mc, bf16x8 *p, float &r0, float &r1) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kb = kk >> 1, i = 2 * (kk & 1) + h;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                p[kk][4 * h + j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[kb][i * 4 + j], x.c, -mc));
            r0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[kk][4 * h], p[kk][4 * h + 1]}, one, r0, false);
            r1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p[kk][4 * h + 2], p[kk][4 * h + 3]}, one, r1, false);
        }
    };
    auto rowmax = [&](const f32x16 *sv) {
        float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                mx0 = fmaxf(fmaxf(mx0, sv[kb][e]), sv[kb][e + 1]);
                mx1 = fmaxf(fmaxf(mx1, sv[kb][e + 2]), sv[kb][e + 3]);
            }
        return xhalf_max(fmaxf(mx0, mx1));
    };
    // Keys at or past kv_end get -inf.  Element 4i + j of block kb is key
    // t0 + 32 kb + 8 i + 4 hw + j: a group of four is tested only if some
    // lane's key in it may be past the end (uniform), against a per-lane
    // limit that is redefined at every call, so that the compiler does not
    // hoist the tests out of the item loop into spilled scalar masks.
    auto mask = [&](int t0, f32x16 *sv) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int rem = x.kv_end - t0 - 32 * kb;   // valid keys of the block
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (8 * i + 7 >= rem) {
                    int lim = rem - 8 * i - 4 * x.hw;
                    asm volatile("" : "+v"(lim));
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (j >= lim) sv[kb][4 * i + j] = -INFINITY;
                }
        }
    };

    // Tile 0: scores and max.
    f32x16 s0[2], s1[2];
    scores<D, NW>(lo, qf, K, s0);
    mask(0, s0);
    st.m = rowmax(s0);
    const float mc = st.m * x.c;

    // Scores of tile 1 beside the probabilities of tile 0 (half a k-step per chunk).
    bf16x8 p0[PS], p1[PS];
    float a0 = 0.f, a1 = 0.f;
    {
        bf16x8 kop[LA + 1][2];
#pragma unroll
        for (int c = 0; c < LA; ++c) read_k(K + TILE, c, kop[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < KS; ++c) {
            if (c + LA < KS) read_k(K + TILE, c + LA, kop[(c + LA) % (LA + 1)]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s1[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[c % (LA + 1)][kb], qf[c],
                                                                 c == 0 ? f32x16{} : s1[kb], 0, 0, 0);
            if (c & 1) prob_step(s0, c >> 1, mc, p0, a0, a1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    mask(BN, s1);
    st.l = a0 + a1;

    // P V of tile 0 beside the probabilities of tile 1 against tile 0's max.
    float b0 = 0.f, b1 = 0.f;
    {
        bf16x8 vop[LA + 1][2];
#pragma unroll
        for (int c = 0; c < LA; ++c) read_v(V, c, vop[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2 * PS; ++c) {
            if (c + LA < 2 * PS) read_v(V, c + LA, vop[(c + LA) % (LA + 1)]);
            const int k = c >> 1, dbp = c & 1;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                st.o[2 * dbp + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[c % (LA + 1)][j], p0[k],
                                                                            c < 2 ? f32x16{} : st.o[2 * dbp + j], 0, 0, 0);
            if (c & 1) prob_step(s1, c >> 1, mc, p1, b0, b1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float rsum = b0 + b1;
    if (__builtin_amdgcn_ballot_w64(!(rsum <= RESCALE_SUM))) {
        const float m_new = fmaxf(st.m, rowmax(s1));
        const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * x.c);
        st.m = m_new;
        st.l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[db][e] *= alpha;
        const float mc1 = m_new * x.c;
        b0 = b1 = 0.f;
#pragma unroll
        for (int k = 0; k < PS; ++k) prob_step(s1, k, mc1, p1, b0, b1);
        rsum = b0 + b1;
    }
    st.l += rsum;

    // P V of tile 1.
    {
        bf16x8 vop[LA + 1][2];
#pragma unroll
        for (int c = 0; c < LA; ++c) read_v(V + TILE, c, vop[c]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2 * PS; ++c) {
            if (c + LA < 2 * PS) read_v(V + TILE, c + LA, vop[(c + LA) % (LA + 1)]);
            const int k = c >> 1, dbp = c & 1;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                st.o[2 * dbp + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[c % (LA + 1)][j], p1[k], st.o[2 * dbp + j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// a2v and audio self-attention have at most a few hundred (audio) keys: a
// workgroup loads all K/V tiles of its head into LDS once (K tiles, then V
// tiles) and then streams a contiguous range of query tiles (32 rows per
// wave) past them.  Q and O move as whole rows: with at most 128 keys
// (STAGED, 8 waves, D = 128) each wave DMAs its 32 query rows into a
// wave-private LDS slot (1 KB = 4 rows per instruction), takes its MFMA
// operands from there, computes with kv2_block, and stages its output rows
// through the same slot for 16-byte-per-lane row stores; the next tile's Q
// is fetched after the stores, the other wave of the SIMD computing
// meanwhile.  Otherwise (more keys, or D = 64) the waves -- 8 at D = 128 for
// long query streams, two per SIMD, else 4 -- take Q straight into
// registers, one tile ahead, and run the tiles one after another.  No
// workgroup barrier is needed except when the head changes.
constexpr int KVRES_SLOT = 32 * 128 * 2;   // one wave's 32 rows of Q or O at D = 128 (8 KB)

template <int D, int NW, bool STAGED, bool GATED, bool QP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2)))
void fa_kvres_kernel(const FaArgs a) {
    constexpr int BM = 32 * NW, KS = D / 16, NDB = D / 32, NKB = BN / 32, PS = BN / 16;
    constexpr int TILE = BN * D * 2;
    constexpr int ROWB = D * 2;             // bytes per Q/O row
    extern __shared__ __attribute__((aligned(1024))) char smem_dyn[];   // [K tiles][V tiles][wave slots]
    LDS_AS char *const lds = (LDS_AS char *)smem_dyn;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hw = lane >> 5, l32 = lane & 31;
    // STAGED holds two tiles (the rows past kv_len read as zeros), else every tile of the keys.
    const int nkt = STAGED ? 2 : (a.kv_len + BN - 1) / BN;
    LDS_AS char *const slot = lds + nkt * 2 * TILE + wave * KVRES_SLOT;   // STAGED: this wave's Q/O rows

    // This workgroup's items: a contiguous share of its group's range (the
    // group is its XCD's contiguous range of items, as in fa_fwd_kernel).
    const int g = blockIdx.x % a.groups, local = blockIdx.x / a.groups;
    const int per_group = gridDim.x / a.groups;
    const int i_begin = g * a.ipg + (int)((int64_t)local * a.ipg / per_group);
    const int i_end = g * a.ipg + (int)((int64_t)(local + 1) * a.ipg / per_group);
    if (i_begin >= i_end) return;   // uniform for the workgroup

    TileCtx x;
    x.kv_end = a.kv_len;
    x.c = a.scale_log2;
    x.wave = wave;
    x.hw = hw;
    x.k_stride = (int)(a.k_ss * 2);
    x.v_stride = (int)(a.v_ss * 2);

    LaneOffsets<D, NW> lo;
#pragma unroll
    for (int n = 0; n < LaneOffsets<D, NW>::PER_THREAD; ++n) {
        const int idx = (n * NW + wave) * 64 + lane;
        const int r = idx / (D / 8), p = idx % (D / 8);
        lo.k_src[n] = r * x.k_stride + swz_k<D>(r, p) * 16;
        lo.v_src[n] = r * x.v_stride + swz_v<D>(r, p) * 16;
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) lo.k_rd[k] = l32 * 2 * D + swz_k<D>(l32, 2 * k + hw) * 16;
    {
        const int li = lane & 15, gg = (lane >> 4) & 1;
        const int r0 = 4 * hw + (li >> 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = 32 * db + 16 * gg + 4 * (li & 3);
            lo.v_rd[db] = r0 * 2 * D + swz_v<D>(r0, col >> 3) * 16 + ((col >> 2) & 1) * 8;
        }
    }

    // Q rows of an item for this wave: STAGED -> DMA of whole rows into a
    // slot (row r of the 32 at r * ROWB, chunks swizzled like K); else
    // straight into the B-operand registers.
    auto q_rsrc = [&](int item) {
        const int bh = item / a.n_qtiles, b = bh / a.H, hh = bh % a.H;
        return make_rsrc(a.q + b * a.q_sb + hh * a.q_sh, ((int64_t)(a.Sq - 1) * a.q_ss + D) * 2);
    };
    auto q_row0 = [&](int item) { return (item % a.n_qtiles) * BM + wave * 32; };
    // STAGED: the 32 rows of this wave's query tile in a [B, Sq, H, D] tensor
    // (Q, the output gate or O) as a buffer resource that starts at the
    // tile's first row; rows at or past Sq lie outside its range (loads read
    // zeros, stores are dropped).  Lane offsets within it, the same for every
    // item: chunk idx = n * 64 + lane of the slot is row idx / (D / 8),
    // physical chunk idx % (D / 8), which holds the row's chunk swz_k of it.
    constexpr int NRC = STAGED ? 32 * (D / 8) / 64 : 1;   // 16-byte chunks per lane
    auto rows_rsrc = [&](int item, const __bf16 *t, int64_t sb, int64_t ss, int64_t sh) {
        const int bh = item / a.n_qtiles, b = bh / a.H, hh = bh % a.H;
        const int r0 = q_row0(item);
        const int64_t bytes = r0 < a.Sq ? ((int64_t)(a.Sq - 1 - r0) * ss + D) * 2 : 0;
        return make_rsrc(t + b * sb + hh * sh + (int64_t)r0 * ss, bytes);
    };
    auto row_offsets = [&](int64_t ss, bool swizzled_src, int *off) {
#pragma unroll
        for (int n = 0; n < NRC; ++n) {
            const int idx = n * 64 + lane;
            const int r = idx / (D / 8), p = idx % (D / 8);
            off[n] = r * (int)(ss * 2) + (swizzled_src ? swz_k<D>(r, p) : p) * 16;
        }
    };
    int q_off[NRC], g_off[GATED ? NRC : 1], o_off[NRC];
    if constexpr (STAGED) {
        row_offsets(a.q_ss, true, q_off);
        if constexpr (GATED) row_offsets(a.g_ss, true, g_off);
        row_offsets(a.o_ss, false, o_off);
    }
    auto dma_rows = [&](int item, LDS_AS char *slot, const __bf16 *t, int64_t sb, int64_t ss, int64_t sh,
                        const int *off) {
        const __amdgpu_buffer_rsrc_t tr = rows_rsrc(item, t, sb, ss, sh);
#pragma unroll
        for (int n = 0; n < NRC; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(tr, (LDS_AS void *)(slot + n * 1024), 16, off[n], 0, 0, 0);
    };
    auto dma_q = [&](int item, LDS_AS char *slot) { dma_rows(item, slot, a.q, a.q_sb, a.q_ss, a.q_sh, q_off); };
    auto regs_q = [&](int item, bf16x8 *qf) {
        const __amdgpu_buffer_rsrc_t qr = q_rsrc(item);
        const int qrow = q_row0(item) + l32;
#pragma unroll
        for (int k = 0; k < KS; ++k)
            qf[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                qr, (int)((int64_t)qrow * a.q_ss * 2) + (2 * k + hw) * 16, 0, 0));
    };

    bf16x8 qf[KS], qn[KS];
    if (STAGED) dma_q(i_begin, slot);
    else regs_q(i_begin, qf);
    int cur_bh = -1;
    for (int item = i_begin; item < i_end; ++item) {
        const int qt = item % a.n_qtiles, bh = item / a.n_qtiles;
        const int b = bh / a.H, hh = bh % a.H;
        if (bh != cur_bh) {   // uniform: load every K/V tile of this head
            __syncthreads();  // all waves are done with the previous head's tiles
            x.kr = make_rsrc(a.k + b * a.k_sb + hh * a.k_sh, ((int64_t)(a.kv_len - 1) * a.k_ss + D) * 2);
            x.vr = make_rsrc(a.v + b * a.v_sb + hh * a.v_sh, ((int64_t)(a.kv_len - 1) * a.v_ss + D) * 2);
            for (int t = 0; t < nkt; ++t) {
                dma_tile<D, NW>(x.kr, lo.k_src, t * BN * x.k_stride, lds + t * TILE, wave);
                dma_tile<D, NW>(x.vr, lo.v_src, t * BN * x.v_stride, lds + (nkt + t) * TILE, wave);
            }
            tile_barrier();   // also completes this wave's Q
            cur_bh = bh;
        }
        if (STAGED) {
            // Q of this item is in `slot` (this wave's own DMA): wait for it
            // and read the B operand; the next item's Q follows the stores.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int k = 0; k < KS; ++k)
                qf[k] = __builtin_bit_cast(bf16x8,
                    *(const LDS_AS u32x4 *)(slot + l32 * ROWB + swz_k<D>(l32, 2 * k + hw) * 16));
            if constexpr (GATED) {   // the gate rows of this tile take Q's place in the slot
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                dma_rows(item, slot, a.g, a.g_sb, a.g_ss, a.g_sh, g_off);
            }
        } else if (item + 1 < i_end) {
            regs_q(item + 1, qn);
        }

        if constexpr (QP) q_prologue<D>(a.qp, qf, min(q_row0(item) + l32, a.Sq - 1), hw);
        RowState<D> st;
#pragma unroll
        for (int i = 0; i < NDB; ++i) st.o[i] = f32x16{};
        st.m = -1e30f;
        st.l = 0.f;
        if constexpr (STAGED) {
            kv2_block<D, NW>(x, lo, qf, lds, lds + 2 * TILE, st);
        } else {
            for (int t = 0; t < nkt; ++t) {
                const LDS_AS char *kt = lds + t * TILE;
                const LDS_AS char *vt = lds + (nkt + t) * TILE;
                f32x16 sc[NKB];
                scores<D, NW>(lo, qf, kt, sc);
                mask_tail(x, t * BN, sc);
                update_max<D>(x, sc, st);
                bf16x8 pf[PS];
                probs<D>(x, sc, st, pf);
                accumulate_pv<D, NW>(lo, vt, pf, st);
            }
        }
        const float inv = 1.0f / xhalf_sum(st.l);
        __bf16 *obase = a.o + b * a.o_sb + hh * a.o_sh;
        const int qrow0 = qt * BM + wave * 32;
        if (STAGED) {
            // O^T fragments -> row-major rows in `slot` (its Q is in registers
            // already), then whole rows out with 16 bytes per lane.
            // Gated: the slot holds the gate rows (loaded during the compute);
            // each lane reads its gate values where its output values go.
            if constexpr (GATED) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = 32 * db + 8 * i + 4 * hw;   // element column of ov[0]
                    LDS_AS bf16x4 *cell = (LDS_AS bf16x4 *)(slot + l32 * ROWB + swz_k<D>(l32, col >> 3) * 16 + (col & 7) * 2);
                    bf16x4 ov;
                    if constexpr (GATED) {
                        const bf16x4 gv = *cell;
#pragma unroll
                        for (int j = 0; j < 4; ++j) ov[j] = (__bf16)((st.o[db][i * 4 + j] * inv) * (float)gv[j]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(st.o[db][i * 4 + j] * inv);
                    }
                    *cell = ov;
                }
            const __amdgpu_buffer_rsrc_t orr = rows_rsrc(item, a.o, a.o_sb, a.o_ss, a.o_sh);
#pragma unroll
            for (int n = 0; n < NRC; ++n) {
                const int idx = n * 64 + lane;
                const int r = idx / (D / 8), c = idx % (D / 8);
                const u32x4 w = *(const LDS_AS u32x4 *)(slot + r * ROWB + swz_k<D>(r, c) * 16);
                __builtin_amdgcn_raw_buffer_store_b128(w, orr, o_off[n], 0, 0);
            }
            if (item + 1 < i_end) {
                // The slot's output rows have been read (the stores hold them); refill it.
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                dma_q(item + 1, slot);
            }
        } else {
            const int qrow = qrow0 + l32;
            if (qrow < a.Sq)
                store_row<NDB>(obase + (int64_t)qrow * a.o_ss,
                               a.g + b * a.g_sb + (int64_t)qrow * a.g_ss + hh * a.g_sh, GATED,
                               st.o, inv, hw);
#pragma unroll
            for (int k = 0; k < KS; ++k) qf[k] = qn[k];
        }
    }
}

// Merge the parts of one output row of a split item: M = max_r m_r,
// L = sum_r l_r 2^(m_r - M), O = sum_r 2^(m_r - M) O_r / L, in part order.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fa_combine_kernel(const CombineArgs a) {
    constexpr int TPR = D / 4;   // threads per output row, 4 floats each
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int BM = a.bm;
    const int64_t row = gt / TPR;           // row of the split items' [item][bm] rows
    const int d4 = (int)(gt % TPR);
    if (row >= (int64_t)a.n_split_items * BM) return;
    const int local = (int)(row / BM), r = (int)(row % BM);   // split index, row in tile
    const int spg = a.ipg - a.wpg;
    const int item = (local / spg) * a.ipg + a.wpg + local % spg;
    const int qt = item % a.n_qtiles, bh = item / a.n_qtiles;
    const int q = qt * BM + r;
    if (q >= a.Sq) return;
    const int b = bh / a.H, hh = bh % a.H;
    const int64_t base = (int64_t)local * a.nsplit * BM + r;
    float M = -INFINITY;
    for (int p = 0; p < a.nsplit; ++p) M = fmaxf(M, a.part_ml[(base + (int64_t)p * BM) * 2]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.nsplit; ++p) {
        const int64_t pr = base + (int64_t)p * BM;
        const float w = __builtin_amdgcn_exp2f(a.part_ml[pr * 2] - M);
        L += w * a.part_ml[pr * 2 + 1];
        const f32x4 ov = *(const f32x4 *)(a.part_o + pr * D + d4 * 4);
        acc += w * ov;
    }
    const float inv = 1.0f / L;
    bf16x4 out;
    if (a.g) {
        const bf16x4 gv = *(const bf16x4 *)(a.g + b * a.g_sb + (int64_t)q * a.g_ss + hh * a.g_sh + d4 * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = (__bf16)((acc[j] * inv) * (float)gv[j]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = (__bf16)(acc[j] * inv);
    }
    *(bf16x4 *)(a.o + b * a.o_sb + (int64_t)q * a.o_ss + hh * a.o_sh + d4 * 4) = out;
}

// ------------------------------------------------------------------ host side

struct Extent {
    uintptr_t lo, hi;
};

// Layout checks of one [B, S, H, D] tensor; its byte range goes to *ext.
// An output must also not map two of its (b, s, h) rows onto the same bytes:
// taking its dimensions of extent > 1 in order of increasing stride, each
// stride must reach past everything the inner dimensions span.
int check_tensor(const ltxattn_tensor &t, int B, int S, int H, int D, bool output, Extent *ext) {
    if (!t.data) return LTXATTN_ERR_INVALID_ARG;
    if ((uintptr_t)t.data % 16) return LTXATTN_ERR_INVALID_ARG;
    if (t.stride_b < 0 || t.stride_s < D || t.stride_h < D) return LTXATTN_ERR_INVALID_ARG;
    if (t.stride_b % 8 || t.stride_s % 8 || t.stride_h % 8) return LTXATTN_ERR_INVALID_ARG;
    // One (batch, head) slice, plus the rows a kernel may touch past the end
    // of it (a query tile and a key tile), must be addressable with 32-bit
    // byte offsets, so that buffer range checks see every such row.
    const int64_t slice = ((int64_t)(S + BM_MAX + BN) * t.stride_s + D) * 2;
    if (slice >= ((int64_t)1 << 31) - 64) return LTXATTN_ERR_UNSUPPORTED;
    if (output) {
        int64_t st[3] = {t.stride_b, t.stride_s, t.stride_h}, ex[3] = {B, S, H};
        for (int i = 0; i < 3; ++i)   // insertion sort by stride
            for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
                std::swap(st[j], st[j - 1]);
                std::swap(ex[j], ex[j - 1]);
            }
        int64_t span = D;   // elements spanned by the dimensions inside the current one
        for (int i = 0; i < 3; ++i) {
            if (ex[i] <= 1) continue;
            if (st[i] < span) return LTXATTN_ERR_INVALID_ARG;
            span += st[i] * (ex[i] - 1);
        }
    }
    const int64_t span = (int64_t)(B - 1) * t.stride_b + (int64_t)(S - 1) * t.stride_s +
                         (int64_t)(H - 1) * t.stride_h + D;
    ext->lo = (uintptr_t)t.data;
    ext->hi = (uintptr_t)t.data + (uintptr_t)span * 2;
    return LTXATTN_OK;
}

bool overlaps(const Extent &x, const Extent &y) { return x.lo < y.hi && y.lo < x.hi; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

constexpr int LONG_ROWS = 1024;   // query and key rows from which 8-wave workgroups are used

constexpr int RESIDENT_KV_MAX = 4 * BN;   // keys held in LDS by fa_kvres_kernel (128 KB)
constexpr size_t LDS_BYTES = 160 * 1024;  // LDS per CU on gfx950

// Workspace of split work items, in rows of [D] fp32 partial O plus 2 fp32
// (m, l).  Region TAIL holds the split last round of video self-attention:
// its split items fill at most one round of workgroups, num_cus * 256 rows
// whatever the kernel (8-wave workgroups of 256 queries, or two 4-wave ones of
// 128 per CU).  Region V2A holds the parts of v2a: items * parts <= num_cus
// by construction, 128 rows each.
enum { REGION_NONE = -1, REGION_TAIL = 0, REGION_V2A = 1 };
// Compute units ltxattn_check_block plans for (no device at hand): MI355X's.
constexpr int CHECK_CUS = 256;
int64_t region_rows(int region, int num_cus) {
    return region == REGION_TAIL ? (int64_t)num_cus * BM_MAX : (int64_t)num_cus * 128;
}

// The launch of one kind, decided on the host before anything is enqueued.
struct Plan {
    const void *kernel = nullptr;   // the attention kernel
    FaArgs a = {};                  // its arguments (part_o / part_ml set at launch)
    int threads = 0;
    size_t lds = 0;                 // dynamic LDS bytes
    int region = REGION_NONE;       // workspace region of the split parts
    int64_t ws_rows = 0;            // rows of that region the parts use
    int bm = 0, n_split_items = 0;  // a combine kernel follows when n_split_items > 0
};

void fill_args(FaArgs &a, const ltxattn_attn_io &io, int B, int H, int D, int Sq, int kv_len) {
    a.q = (const __bf16 *)io.q.data;
    a.k = (const __bf16 *)io.k.data;
    a.v = (const __bf16 *)io.v.data;
    a.q_sb = io.q.stride_b; a.q_ss = io.q.stride_s; a.q_sh = io.q.stride_h;
    a.k_sb = io.k.stride_b; a.k_ss = io.k.stride_s; a.k_sh = io.k.stride_h;
    a.v_sb = io.v.stride_b; a.v_ss = io.v.stride_s; a.v_sh = io.v.stride_h;
    a.o = (__bf16 *)io.o.data;
    a.o_sb = io.o.stride_b; a.o_ss = io.o.stride_s; a.o_sh = io.o.stride_h;
    a.g = (const __bf16 *)io.gate.data;
    a.g_sb = io.gate.stride_b; a.g_ss = io.gate.stride_s; a.g_sh = io.gate.stride_h;
    a.B = B; a.H = H; a.Sq = Sq; a.kv_len = kv_len;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const ltxattn_qk_prologue &pro = io.prologue;
    if (pro.q_weight)
        a.qp = QkPrologue{pro.q_weight, pro.q_cos, pro.q_sin, pro.eps, pro.pairing == LTXATTN_ROPE_INTERLEAVED};
}

// The resident-key kernel's instantiation.  Gated outputs and the query
// prologue take instantiations of their own, so that the plain one is
// compiled without any of their code (a uniform branch in its item loop
// costs registers the staged variant does not have).
template <int D, int NW, bool ST>
const void *kvres_variant(bool gated, bool qp) {
    if (gated)
        return qp ? (const void *)&fa_kvres_kernel<D, NW, ST, true, true> : (const void *)&fa_kvres_kernel<D, NW, ST, true, false>;
    return qp ? (const void *)&fa_kvres_kernel<D, NW, ST, false, true> : (const void *)&fa_kvres_kernel<D, NW, ST, false, false>;
}

const void *kvres_kernel(int D, int nw, bool staged, bool gated, bool qp) {
    if (D == 128 && staged) return kvres_variant<128, 8, true>(gated, qp);
    if (D == 128 && nw == 8) return kvres_variant<128, 8, false>(gated, qp);
    if (D == 128) return kvres_variant<128, 4, false>(gated, qp);
    return kvres_variant<64, 4, false>(gated, qp);
}

// a2v and audio self-attention: all keys resident in LDS, query tiles streamed.
Plan plan_resident_kv(int num_cus, int H, int D, const ltxattn_attn_io &io, int B, int Sq, int kv_len) {
    Plan p;
    FaArgs &a = p.a;
    fill_args(a, io, B, H, D, Sq, kv_len);
    const int nkt = ceil_div(kv_len, BN);
    const size_t kv_lds = (size_t)nkt * 2 * BN * D * 2;
    // D = 128: 8 waves, two per SIMD, with Q and O rows staged through one
    // 8 KB slot per wave and the two-tile pass when there are at most 128
    // keys, else with Q straight from HBM into registers (up to 256 keys:
    // 128 KB of K/V) -- or 4 such waves when 256-query items would leave
    // most CUs idle (a short query stream such as audio self-attention).
    // D = 64: 4 unstaged waves.
    const bool staged = D == 128 && nkt <= 2;
    const int nw = staged || (D == 128 && (int64_t)B * H * ceil_div(Sq, 256) >= num_cus) ? 8 : 4;
    p.lds = staged ? (size_t)2 * 2 * BN * D * 2 + (size_t)8 * KVRES_SLOT : kv_lds;
    a.n_qtiles = ceil_div(Sq, 32 * nw);
    const int items = B * H * a.n_qtiles;
    const int per_cu = (int)std::min<size_t>(2, LDS_BYTES / p.lds);   // LDS-resident workgroups per CU
    a.groups = (items % 8 == 0 && num_cus % 8 == 0) ? 8 : 1;
    a.ipg = items / a.groups;
    const int per_group = std::min(a.ipg, (nw == 8 ? 1 : per_cu) * num_cus / a.groups);
    a.total = a.groups * per_group;
    p.threads = 64 * nw;
    p.kernel = kvres_kernel(D, nw, staged, a.g != nullptr, a.qp.w != nullptr);
    return p;
}

// v2a: one workgroup per CU streams one key range of one 128-query item
// (fa_ring_kernel with two key groups); as many ranges per item as fill the CUs.
Plan plan_stream(int num_cus, int H, int D, const ltxattn_attn_io &io, int B, int Sq, int kv_len) {
    Plan p;
    FaArgs &a = p.a;
    fill_args(a, io, B, H, D, Sq, kv_len);
    const int BM = 128;
    a.n_qtiles = ceil_div(Sq, BM);
    const int items = B * H * a.n_qtiles;
    a.groups = (items % 8 == 0 && num_cus % 8 == 0) ? 8 : 1;
    a.ipg = items / a.groups;
    // Parts per item: one workgroup per CU, at most NSPLIT_MAX, at least
    // four key tiles per part.
    int ns = num_cus / items;
    ns = ns < NSPLIT_MAX ? ns : NSPLIT_MAX;
    const int by_len = kv_len / (4 * BN);
    ns = ns < by_len ? ns : by_len;
    ns = ns < 1 ? 1 : ns;
    a.split_len = ceil_div(ceil_div(kv_len, ns), BN) * BN;
    ns = ceil_div(kv_len, a.split_len);    // every part holds at least one key
    a.nsplit = ns;
    a.wpg = ns == 1 ? a.ipg : 0;           // one part: every item is whole
    a.total = items * ns;
    p.threads = 64 * RING_NW;
    p.lds = (size_t)RING_STAGES * 2 * BN * D * 2;
    const bool qp = a.qp.w != nullptr;
    p.kernel = D == 128 ? (qp ? (const void *)&fa_ring_kernel<128, RING_NW, 2, true> : (const void *)&fa_ring_kernel<128, RING_NW, 2>)
                        : (qp ? (const void *)&fa_ring_kernel<64, RING_NW, 2, true> : (const void *)&fa_ring_kernel<64, RING_NW, 2>);
    if (ns > 1) {
        p.region = REGION_V2A;
        p.ws_rows = (int64_t)items * ns * BM;
        p.bm = BM;
        p.n_split_items = items;
    }
    return p;
}

// One kind's launch.  v2a takes the split-KV stream; a short key stream the
// resident-key kernel; otherwise the ring kernel (long query and key
// streams at D = 128: 256-query workgroups, so each K/V tile is fetched
// once per 256 queries) or fa_fwd_kernel (128 queries).  With tail_split,
// the items of an incomplete last round may run as key-range parts in the
// TAIL region; only video self-attention does this, so that no other kind
// shares that region with it when the audio side runs on its own stream.
Plan plan_kind(int num_cus, int H, int D, const ltxattn_attn_io &io, int B, int Sq, int kv_len,
               bool split_all, bool tail_split) {
    if (split_all) return plan_stream(num_cus, H, D, io, B, Sq, kv_len);
    if (kv_len <= RESIDENT_KV_MAX) return plan_resident_kv(num_cus, H, D, io, B, Sq, kv_len);
    Plan p;
    FaArgs &a = p.a;
    fill_args(a, io, B, H, D, Sq, kv_len);
    const int NW = (Sq >= LONG_ROWS && kv_len >= LONG_ROWS && D == 128) ? 8 : 4;
    const int BM = 32 * NW;
    a.n_qtiles = ceil_div(Sq, BM);
    const int items = B * H * a.n_qtiles;
    // One group per XCD when the items divide evenly, else a single group.
    const int groups = (items % 8 == 0 && num_cus % 8 == 0) ? 8 : 1;
    const int ipg = items / groups;
    const int slots = WAVES_PER_CU / NW * num_cus / groups;   // workgroups resident per group
    int spg = 0, ns = 1;                                 // split items per group, parts each
    if (tail_split && ipg > slots) {
        // Split the items of an incomplete last round so that it fills its XCD.
        const int rem = ipg % slots;
        if (rem > 0 && 2 * rem <= slots) {
            ns = slots / rem;
            ns = ns < NSPLIT_MAX ? ns : NSPLIT_MAX;
            const int by_len = kv_len / (4 * BN);
            ns = ns < by_len ? ns : by_len;
            if (ns > 1) spg = rem;
        }
    }
    if (spg == 0) ns = 1;
    a.split_len = ceil_div(ceil_div(kv_len, ns), BN) * BN;
    ns = ceil_div(kv_len, a.split_len);   // every part holds at least one key
    if (ns == 1) spg = 0;
    a.nsplit = ns;
    a.groups = groups;
    a.ipg = ipg;
    a.wpg = ipg - spg;
    // Two parts per split item on exactly half of each group's CUs: deal
    // them first and last (measured: 0.4-1% off the video kernel).
    a.stagger = D == 128 && NW == 8 && ns == 2 && 2 * spg == slots;
    a.total = groups * (a.wpg + spg * ns);
    const int n_split_items = groups * spg;
    if (n_split_items > 0) {
        p.region = REGION_TAIL;
        p.ws_rows = (int64_t)n_split_items * ns * BM;
        p.bm = BM;
        p.n_split_items = n_split_items;
    }
    if (D == 128 && NW == 8) {
        p.kernel = a.qp.w ? (const void *)&fa_ring_kernel<128, RING_NW, 1, true> : (const void *)&fa_ring_kernel<128, RING_NW, 1>;
        p.threads = 64 * RING_NW;
        p.lds = (size_t)RING_STAGES * 2 * BN * 128 * 2;
    } else {
        p.kernel = D == 128 ? (const void *)&fa_fwd_kernel<128, 4> : (const void *)&fa_fwd_kernel<64, 4>;
        p.threads = 256;
    }
    return p;
}

// Launch order of the kinds.  v2a runs straight after video self-attention:
// it streams the same video K and V, part of which the last-level cache
// still holds; a2v, which writes a video-sized output, comes after it.
constexpr int KIND_ORDER[4] = {LTXATTN_VIDEO_SELF, LTXATTN_V2A, LTXATTN_A2V, LTXATTN_AUDIO_SELF};

// The plan of every kind whose output is given (on[k]) for a device with
// num_cus compute units.
void plan_block(const ltxattn_config &caps, const ltxattn_block_io *io, const bool on[4], int num_cus,
                Plan plans[4]) {
    const int B = io->batch, Sv = io->video_len, La = io->audio_len, Lk = io->audio_kv_len;
    const int q_rows[4] = {Sv, La, Sv, La};
    for (int k = 0; k < 4; ++k) {
        if (!on[k]) continue;
        const int kv_len = (k == LTXATTN_AUDIO_SELF || k == LTXATTN_A2V) ? Lk : Sv;
        plans[k] = plan_kind(num_cus, caps.heads, caps.head_dim, io->attn[k], B, q_rows[k], kv_len,
                             k == LTXATTN_V2A, k == LTXATTN_VIDEO_SELF);
    }
}

// The prologue of one kind: every pointer given and 16-byte aligned, eps a
// positive number, a known pairing.
int check_prologue(const ltxattn_qk_prologue &p) {
    const void *ptrs[6] = {p.q_weight, p.k_weight, p.q_cos, p.q_sin, p.k_cos, p.k_sin};
    for (const void *q : ptrs)
        if (!q || (uintptr_t)q % 16) return LTXATTN_ERR_INVALID_ARG;
    if (!(p.eps > 0.f) || !std::isfinite(p.eps)) return LTXATTN_ERR_INVALID_ARG;
    if (p.pairing != LTXATTN_ROPE_HALF && p.pairing != LTXATTN_ROPE_INTERLEAVED) return LTXATTN_ERR_INVALID_ARG;
    return LTXATTN_OK;
}

bool has_prologue(const ltxattn_block_io *io, int k) { return io->attn[k].prologue.q_weight != nullptr; }

// One prologue pass over a kind's keys, into a slot of the key workspace.
struct KeyPass {
    PrologueRowsArgs a;
    int blocks;
};

// The key workspace: slots 0 and 1 hold video-sized keys, 2 and 3
// audio-sized ones, each [batch][rows][heads][head_dim] bf16.
struct KeyWorkspace {
    __bf16 *base;
    int64_t video_elems, audio_elems;   // per slot
    __bf16 *slot(int i) const { return base + (i < 2 ? i * video_elems : 2 * video_elems + (i - 2) * audio_elems); }
};

// The key passes of a call, and each prologue kind's plan pointed at its
// prepared keys.  Kinds whose keys are the same tensor under the same k
// parameters share one pass.  Video keys (video self, v2a) take slots 0-1,
// audio keys (audio self, a2v) slots 2-3.
int plan_key_passes(const ltxattn_block_io *io, const bool on[4], int H, int D, const KeyWorkspace &kw,
                    Plan plans[4], KeyPass passes[4]) {
    int n = 0, slot_of[4] = {-1, -1, -1, -1}, next[2] = {0, 2};
    const int B = io->batch;
    for (int k = 0; k < 4; ++k) {
        if (!on[k] || !has_prologue(io, k)) continue;
        const bool video = k == LTXATTN_VIDEO_SELF || k == LTXATTN_V2A;
        const int S = video ? io->video_len : io->audio_len;
        const ltxattn_tensor &kt = io->attn[k].k;
        const ltxattn_qk_prologue &p = io->attn[k].prologue;
        int slot = -1;
        for (int j = 0; j < k && slot < 0; ++j) {
            if (slot_of[j] < 0 || (j == LTXATTN_VIDEO_SELF || j == LTXATTN_V2A) != video) continue;
            const ltxattn_tensor &jt = io->attn[j].k;
            const ltxattn_qk_prologue &q = io->attn[j].prologue;
            if (jt.data == kt.data && jt.stride_b == kt.stride_b && jt.stride_s == kt.stride_s &&
                jt.stride_h == kt.stride_h && q.k_weight == p.k_weight && q.k_cos == p.k_cos &&
                q.k_sin == p.k_sin && q.eps == p.eps && q.pairing == p.pairing)
                slot = slot_of[j];
        }
        if (slot < 0) {
            slot = next[video ? 0 : 1]++;
            KeyPass &kp = passes[n++];
            kp.a.x = (const __bf16 *)kt.data;
            kp.a.x_sb = kt.stride_b; kp.a.x_ss = kt.stride_s; kp.a.x_sh = kt.stride_h;
            kp.a.y = kw.slot(slot);
            kp.a.p = QkPrologue{p.k_weight, p.k_cos, p.k_sin, p.eps, p.pairing == LTXATTN_ROPE_INTERLEAVED};
            kp.a.S = S;
            kp.a.H = H;
            kp.a.tokens = (int64_t)B * S;   // one wave per token
            kp.blocks = (int)std::min<int64_t>((kp.a.tokens + 3) / 4, 16384);
        }
        slot_of[k] = slot;
        FaArgs &a = plans[k].a;
        a.k = kw.slot(slot);
        a.k_ss = (int64_t)H * D;
        a.k_sh = D;
        a.k_sb = (int64_t)S * H * D;
    }
    return n;
}

// Argument checks shared by ltxattn_check_block and the block calls, then
// the workspace each kind's split parts need against the rows a workspace
// for num_cus compute units has per region.  on[k] is set for the kinds
// whose output pointer is non-null.
int validate_block(const ltxattn_config &caps, const ltxattn_block_io *io, int num_cus, bool on[4]) {
    const int B = io->batch, Sv = io->video_len, La = io->audio_len, Lk = io->audio_kv_len;
    if (B < 1 || B > caps.max_batch) return LTXATTN_ERR_INVALID_ARG;
    if (Sv < 1 || Sv > caps.max_video_len) return LTXATTN_ERR_INVALID_ARG;
    if (La < 1 || La > caps.max_audio_len) return LTXATTN_ERR_INVALID_ARG;
    if (Lk < 1 || Lk > La) return LTXATTN_ERR_INVALID_ARG;
    const int H = caps.heads, D = caps.head_dim;
    // Rows of q/o and of k/v per kind.
    const int q_rows[4] = {Sv, La, Sv, La};
    const int kv_rows[4] = {Sv, La, La, Sv};
    Extent in_ext[4][4] = {}, out_ext[4];
    for (int k = 0; k < 4; ++k) {
        const ltxattn_attn_io &x = io->attn[k];
        on[k] = x.o.data != nullptr;
        if (!on[k]) continue;
        int rc;
        if ((rc = check_tensor(x.q, B, q_rows[k], H, D, false, &in_ext[k][0]))) return rc;
        if ((rc = check_tensor(x.k, B, kv_rows[k], H, D, false, &in_ext[k][1]))) return rc;
        if ((rc = check_tensor(x.v, B, kv_rows[k], H, D, false, &in_ext[k][2]))) return rc;
        if ((rc = check_tensor(x.o, B, q_rows[k], H, D, true, &out_ext[k]))) return rc;
        if (x.gate.data && (rc = check_tensor(x.gate, B, q_rows[k], H, D, false, &in_ext[k][3]))) return rc;
        if (has_prologue(io, k)) {
            if ((rc = check_prologue(x.prologue))) return rc;
            if (!caps.qk_prologue) return LTXATTN_ERR_UNSUPPORTED;
        }
    }
    for (int k = 0; k < 4; ++k) {
        if (!on[k]) continue;
        for (int j = 0; j < 4; ++j) {
            if (!on[j]) continue;
            for (int t = 0; t < 4; ++t)   // q, k, v, gate (an absent gate spans nothing)
                if (overlaps(out_ext[k], in_ext[j][t])) return LTXATTN_ERR_INVALID_ARG;
            if (j != k && overlaps(out_ext[k], out_ext[j])) return LTXATTN_ERR_INVALID_ARG;
        }
    }
    Plan plans[4];
    plan_block(caps, io, on, num_cus, plans);
    for (int k = 0; k < 4; ++k)
        if (on[k] && plans[k].region != REGION_NONE && plans[k].ws_rows > region_rows(plans[k].region, num_cus))
            return LTXATTN_ERR_UNSUPPORTED;
    return LTXATTN_OK;
}

// The workspace of split parts: two regions, TAIL then V2A, of rows[r] rows
// each, as [rows][D] fp32 partial outputs in o and [rows][2] fp32 (m, l) in ml.
struct Workspace {
    float *o, *ml;
    int64_t rows[2];
};

}  // namespace

struct ltxattn_handle {
    int device;
    int heads, head_dim, max_batch, max_video_len, max_audio_len, qk_prologue;
    int num_cus;
    // Workspace of split items (hipMalloc at create), in two regions so that
    // v2a can run beside video self-attention.
    Workspace ws;
    // Keys prepared by the QK-norm + rotary prologue (qk_prologue only).
    KeyWorkspace kw;
    // ltxattn_block_attention_overlap: the stream the audio-side kinds run
    // on, and the events that fork it from and join it to the caller's.
    hipStream_t side;
    hipEvent_t fork, join;
    int last_hip_error;
    // profiling: PROF_EVENTS events per call, and which of them bound what
    hipEvent_t *events;
    struct ProfCall {
        int8_t start[4], mid[4], end[4];   // per kind; mid < 0: no combine kernel followed;
                                           // start < 0: kind not recorded
        int8_t first, last;                // the whole call (first < 0: not recorded)
        int8_t sync;                       // the call's last recorded event
    } *prof_calls;
    int prof_max, prof_n;
    unsigned prof_kinds;                   // bit k: kind k is recorded
};

namespace {

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            changed = (err == hipSuccess);
        }
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

// hipError_t of the last failed call without a handle to keep it in
// (ltxattn_create, ltxattn_block_attention_noalloc) on this thread.
thread_local int g_create_hip_error = 0;

int hip_fail(ltxattn_handle *h, hipError_t e) {
    if (h) h->last_hip_error = (int)e;
    else g_create_hip_error = (int)e;
    return LTXATTN_ERR_HIP;
}

// Kernels that take more dynamic LDS than the default limit: the resident-key
// kernel keeps up to RESIDENT_KV_MAX keys of K and V (and, staged, the Q/O row
// slots) in LDS, the ring kernels four K/V tile pairs.  For the current device.
hipError_t set_kernel_lds_limits() {
    hipError_t e = hipSuccess;
    for (int v = 0; v < 16 && e == hipSuccess; ++v) {   // (D, waves, staged) x gated x prologue
        const int shape = v >> 2;
        e = hipFuncSetAttribute(kvres_kernel(shape == 3 ? 64 : 128, shape == 2 ? 4 : 8, shape == 0, v & 1, v & 2),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    }
    const void *ring[6] = {(const void *)&fa_ring_kernel<128, RING_NW, 2>, (const void *)&fa_ring_kernel<128, RING_NW, 2, true>,
                           (const void *)&fa_ring_kernel<128, RING_NW, 1>, (const void *)&fa_ring_kernel<128, RING_NW, 1, true>,
                           (const void *)&fa_ring_kernel<64, RING_NW, 2>, (const void *)&fa_ring_kernel<64, RING_NW, 2, true>};
    for (int i = 0; i < 6 && e == hipSuccess; ++i)
        e = hipFuncSetAttribute(ring[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                RING_STAGES * 2 * BN * (i < 4 ? 128 : 64) * 2);
    return e;
}

// Launch one planned kind on stream st, with its split parts (if any) in
// its region of ws, then the combine kernel that merges them.  When
// `after_main` is given and a combine kernel follows, the event is recorded
// between the two and *mid_recorded is set.
int launch_plan(ltxattn_handle *h, int D, const Plan &p, const Workspace &ws, hipStream_t st, hipEvent_t after_main,
                bool *mid_recorded) {
    FaArgs a = p.a;
    if (p.region != REGION_NONE) {
        const int64_t r0 = p.region == REGION_V2A ? ws.rows[REGION_TAIL] : 0;
        a.part_o = ws.o + r0 * D;
        a.part_ml = ws.ml + r0 * 2;
    }
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(p.kernel, dim3(a.total), dim3(p.threads), args, p.lds, st);
    if (e != hipSuccess) return hip_fail(h, e);
    if (p.n_split_items == 0) return LTXATTN_OK;
    if (after_main) {
        if ((e = hipEventRecord(after_main, st)) != hipSuccess) return hip_fail(h, e);
        *mid_recorded = true;
    }
    // Merge the key-range parts of the split items (fa_combine_kernel).
    CombineArgs c;
    c.part_o = a.part_o; c.part_ml = a.part_ml;
    c.o = a.o; c.o_sb = a.o_sb; c.o_ss = a.o_ss; c.o_sh = a.o_sh;
    c.g = a.g; c.g_sb = a.g_sb; c.g_ss = a.g_ss; c.g_sh = a.g_sh;
    c.H = a.H; c.Sq = a.Sq; c.bm = p.bm; c.n_qtiles = a.n_qtiles; c.ipg = a.ipg; c.wpg = a.wpg;
    c.n_split_items = p.n_split_items; c.nsplit = a.nsplit;
    const int64_t threads = (int64_t)p.n_split_items * p.bm * (D / 4);
    void *cargs[] = {&c};
    e = hipLaunchKernel(D == 128 ? (const void *)&fa_combine_kernel<128> : (const void *)&fa_combine_kernel<64>,
                        dim3(ceil_div(threads, 256)), dim3(256), cargs, 0, st);
    return e == hipSuccess ? LTXATTN_OK : hip_fail(h, e);
}

// The block call.  Every argument and the workspace of every kind are
// checked, and every kind planned, before anything is enqueued.  Kinds run
// in KIND_ORDER on the caller's stream; with `overlap`, the audio-side kinds
// (v2a, a2v, audio self) run on the handle's side stream instead, forked
// from the caller's stream at the start of the call and joined back into it
// at the end, so the call stays one ordered unit on the caller's stream (and
// can be captured into a HIP graph from it).  Profiling events, if on, are
// recorded in enqueue order and indexed per call by ProfCall: the call's
// start and end (when every kind is recorded), and for each recorded kind
// its start, the end of its attention kernel when a combine kernel follows,
// and its end, on the stream that runs it.
int enqueue_block(ltxattn_handle *h, const ltxattn_block_io *io, hipStream_t st, bool overlap) {
    if (!h || !io) return LTXATTN_ERR_INVALID_ARG;
    const ltxattn_config caps = {h->device, h->heads, h->head_dim, h->max_batch, h->max_video_len,
                                 h->max_audio_len, h->qk_prologue};
    bool on[4];
    const int vrc = validate_block(caps, io, h->num_cus, on);
    if (vrc) return vrc;
    Plan plans[4];
    plan_block(caps, io, on, h->num_cus, plans);
    KeyPass passes[4];
    const int n_passes = plan_key_passes(io, on, h->heads, h->head_dim, h->kw, plans, passes);

    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return hip_fail(h, g.err);
    // Profiling events go only where something starts or ends: a kind that
    // follows another on the same stream starts at that kind's end event, and
    // a sequential call ends at its last kind's.
    hipEvent_t *ev = nullptr;
    ltxattn_handle::ProfCall *pc = nullptr;
    if (h->events && h->prof_n < h->prof_max) {
        ev = h->events + (int64_t)h->prof_n * PROF_EVENTS;
        pc = h->prof_calls + h->prof_n;
        ++h->prof_n;
    }
    int n_ev = 0;
    hipError_t e = hipSuccess;
    auto record = [&](hipStream_t s) {   // the index of a newly recorded event
        if (e == hipSuccess) e = hipEventRecord(ev[n_ev], s);
        return (int8_t)n_ev++;
    };
    // With every kind recorded the call's own first and last events are
    // kept as well (its total); with a subset only those kinds' boundaries.
    const bool all = h->prof_kinds == 0xFu;
    int8_t last_main = -1, last_side = -1;
    if (ev) pc->first = last_main = all ? record(st) : (int8_t)-1;
    // The prologue passes over keys come first, on the caller's stream, so
    // that both sides of the overlapped call find their keys prepared.
    for (int i = 0; i < n_passes; ++i) {
        void *args[] = {&passes[i].a};
        if (e == hipSuccess)
            e = hipLaunchKernel(h->head_dim == 128 ? (const void *)&qk_prologue_kernel<128>
                                                   : (const void *)&qk_prologue_kernel<64>,
                                dim3(passes[i].blocks), dim3(256), args, 0, st);
    }
    if (ev && n_passes > 0 && all) last_main = record(st);   // the first kind starts after them
    if (overlap) {
        if (e == hipSuccess) e = hipEventRecord(h->fork, st);
        if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork, 0);
    }
    if (e != hipSuccess) return hip_fail(h, e);
    for (int n = 0; n < 4; ++n) {
        const int k = KIND_ORDER[n];
        const bool main = !overlap || k == LTXATTN_VIDEO_SELF;
        hipStream_t ks = main ? st : h->side;
        int8_t &last = main ? last_main : last_side;
        const bool rec_k = ev && (h->prof_kinds >> k & 1u);
        if (ev) {
            pc->start[k] = rec_k ? (last >= 0 ? last : record(ks)) : (int8_t)-1;
            pc->mid[k] = -1;
            pc->end[k] = pc->start[k];
            if (rec_k) last = pc->start[k];
        }
        if (e != hipSuccess) return hip_fail(h, e);
        if (!on[k]) continue;
        bool mid_rec = false;
        const int rc = launch_plan(h, h->head_dim, plans[k], h->ws, ks, rec_k ? ev[n_ev] : nullptr,
                                   rec_k ? &mid_rec : nullptr);
        if (rc) return rc;
        if (rec_k) {
            if (mid_rec) pc->mid[k] = (int8_t)n_ev++;
            pc->end[k] = last = record(ks);
            if (e != hipSuccess) return hip_fail(h, e);
        } else {
            last = -1;   // an unrecorded kind ran since: the next kind records its own start
        }
    }
    if (overlap) {
        if ((e = hipEventRecord(h->join, h->side)) != hipSuccess) return hip_fail(h, e);
        if ((e = hipStreamWaitEvent(st, h->join, 0)) != hipSuccess) return hip_fail(h, e);
    }
    if (ev) {
        pc->last = !all ? (int8_t)-1 : overlap ? record(st) : last_main;
        pc->sync = (int8_t)(n_ev - 1);
        if (e != hipSuccess) return hip_fail(h, e);
    }
    return LTXATTN_OK;
}

// Frees what create allocated (null members are skipped) and the handle;
// returns the first error.
hipError_t release(ltxattn_handle *h) {
    hipError_t first = hipSuccess;
    auto keep = [&](hipError_t e) { if (first == hipSuccess && e != hipSuccess) first = e; };
    if (h->join) keep(hipEventDestroy(h->join));
    if (h->fork) keep(hipEventDestroy(h->fork));
    if (h->side) keep(hipStreamDestroy(h->side));
    if (h->kw.base) keep(hipFree(h->kw.base));
    if (h->ws.ml) keep(hipFree(h->ws.ml));
    if (h->ws.o) keep(hipFree(h->ws.o));
    free(h);
    return first;
}

}  // namespace

// ------------------------------------------------- allocation-free block call
// ltxattn_block_attention_noalloc keeps its split parts in this file-scope
// device array instead of a handle's workspace.  Each device holds its own
// copy from the library's first use on it until the process ends.  In host
// code `scratch` only stands in for the symbol: its address on a device comes
// from hipGetSymbolAddress, taken once per device at that device's set-up.
constexpr int64_t SCRATCH_BYTES = (int64_t)64 << 20;
static __device__ __align__(256) float scratch[SCRATCH_BYTES / 4];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;

struct NoallocDevice {
    float *scratch;   // this device's copy of `scratch`; null until set up
    int num_cus;
};
std::mutex g_noalloc_mutex;
NoallocDevice g_noalloc[NOALLOC_MAX_DEVICES];

// Set-up of the current device, once: its CU count, the kernels' LDS limits
// and the device address of `scratch`.
int noalloc_device(int device, NoallocDevice *out) {
    std::lock_guard<std::mutex> lock(g_noalloc_mutex);
    NoallocDevice &d = g_noalloc[device];
    if (!d.scratch) {
        int num_cus = 0;
        hipError_t e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, device);
        if (e == hipSuccess) e = set_kernel_lds_limits();
        void *ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e == hipSuccess && !ptr) e = hipErrorInvalidSymbol;
        if (e != hipSuccess) return hip_fail(nullptr, e);
        d.num_cus = num_cus;
        d.scratch = (float *)ptr;
    }
    *out = d;
    return LTXATTN_OK;
}

}  // namespace

extern "C" {

const char *ltxattn_status_string(int status) {
    switch (status) {
        case LTXATTN_OK: return "ok";
        case LTXATTN_ERR_INVALID_ARG: return "invalid argument";
        case LTXATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case LTXATTN_ERR_HIP: return "HIP runtime error";
        case LTXATTN_ERR_OOM: return "device workspace allocation failed";
        case LTXATTN_ERR_SCRATCH: return "split parts need more than the static scratch of the allocation-free call";
        default: return "unknown status";
    }
}

int ltxattn_create(const ltxattn_config *cfg, ltxattn_handle **out) {
    if (!out) return LTXATTN_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg) return LTXATTN_ERR_INVALID_ARG;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return LTXATTN_ERR_UNSUPPORTED;
    if (cfg->heads < 1) return LTXATTN_ERR_UNSUPPORTED;
    if (cfg->max_batch < 1 || cfg->max_video_len < 1 || cfg->max_audio_len < 1 || cfg->device < 0)
        return LTXATTN_ERR_INVALID_ARG;
    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess) { g_create_hip_error = (int)e; return LTXATTN_ERR_HIP; }
    if (cfg->device >= ndev) return LTXATTN_ERR_INVALID_ARG;

    ltxattn_handle *h = (ltxattn_handle *)calloc(1, sizeof(ltxattn_handle));
    if (!h) return LTXATTN_ERR_OOM;
    h->device = cfg->device;
    h->heads = cfg->heads;
    h->head_dim = cfg->head_dim;
    h->max_batch = cfg->max_batch;
    h->max_video_len = cfg->max_video_len;
    h->max_audio_len = cfg->max_audio_len;
    h->qk_prologue = cfg->qk_prologue != 0;

    DeviceGuard g(h->device);
    if (g.err != hipSuccess) { g_create_hip_error = (int)g.err; free(h); return LTXATTN_ERR_HIP; }
    e = hipDeviceGetAttribute(&h->num_cus, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) { g_create_hip_error = (int)e; free(h); return LTXATTN_ERR_HIP; }
    e = set_kernel_lds_limits();
    if (e != hipSuccess) { g_create_hip_error = (int)e; free(h); return LTXATTN_ERR_HIP; }
    // Workspace of the split items: both regions at their bounds for this
    // device's compute units.
    h->ws.rows[REGION_TAIL] = region_rows(REGION_TAIL, h->num_cus);
    h->ws.rows[REGION_V2A] = region_rows(REGION_V2A, h->num_cus);
    const int64_t rows = h->ws.rows[REGION_TAIL] + h->ws.rows[REGION_V2A];
    int status = LTXATTN_OK;
    e = hipMalloc((void **)&h->ws.o, (size_t)rows * h->head_dim * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void **)&h->ws.ml, (size_t)rows * 2 * sizeof(float));
    if (e == hipSuccess && h->qk_prologue) {
        const int64_t row = (int64_t)h->heads * h->head_dim;
        h->kw.video_elems = (int64_t)h->max_batch * h->max_video_len * row;
        h->kw.audio_elems = (int64_t)h->max_batch * h->max_audio_len * row;
        e = hipMalloc((void **)&h->kw.base, (size_t)(2 * h->kw.video_elems + 2 * h->kw.audio_elems) * 2);
    }
    if (e != hipSuccess) status = LTXATTN_ERR_OOM;
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->join, hipEventDisableTiming);
    if (e != hipSuccess) {
        g_create_hip_error = (int)e;
        (void)hipGetLastError();
        (void)release(h);   // the failure above is the one reported
        return status ? status : LTXATTN_ERR_HIP;
    }
    *out = h;
    return LTXATTN_OK;
}

int ltxattn_destroy(ltxattn_handle *h) {
    if (!h) return LTXATTN_OK;
    DeviceGuard g(h->device);
    if (h->events) ltxattn_profile_end(h);
    return release(h) == hipSuccess ? LTXATTN_OK : LTXATTN_ERR_HIP;
}

int ltxattn_last_hip_error(const ltxattn_handle *h) { return h ? h->last_hip_error : g_create_hip_error; }

int ltxattn_check_block(const ltxattn_config *cfg, const ltxattn_block_io *io) {
    if (!cfg || !io) return LTXATTN_ERR_INVALID_ARG;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return LTXATTN_ERR_UNSUPPORTED;
    if (cfg->heads < 1) return LTXATTN_ERR_UNSUPPORTED;
    bool on[4];
    return validate_block(*cfg, io, CHECK_CUS, on);
}

int ltxattn_block_attention(ltxattn_handle *h, const ltxattn_block_io *io, void *hip_stream) {
    return enqueue_block(h, io, (hipStream_t)hip_stream, false);
}

int ltxattn_block_attention_overlap(ltxattn_handle *h, const ltxattn_block_io *io, void *hip_stream) {
    return enqueue_block(h, io, (hipStream_t)hip_stream, true);
}

int ltxattn_block_attention_noalloc(const ltxattn_config *cfg, const ltxattn_block_io *io, void *hip_stream) {
    if (!cfg || !io) return LTXATTN_ERR_INVALID_ARG;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return LTXATTN_ERR_UNSUPPORTED;
    if (cfg->heads < 1) return LTXATTN_ERR_UNSUPPORTED;
    if (cfg->max_batch < 1 || cfg->max_video_len < 1 || cfg->max_audio_len < 1 || cfg->device < 0 ||
        cfg->device >= NOALLOC_MAX_DEVICES)
        return LTXATTN_ERR_INVALID_ARG;
    int ndev = 0;
    hipError_t e = hipGetDeviceCount(&ndev);
    if (e != hipSuccess) return hip_fail(nullptr, e);
    if (cfg->device >= ndev) return LTXATTN_ERR_INVALID_ARG;
    DeviceGuard g(cfg->device);
    if (g.err != hipSuccess) return hip_fail(nullptr, g.err);
    NoallocDevice dev;
    int rc = noalloc_device(cfg->device, &dev);
    if (rc) return rc;
    ltxattn_config caps = *cfg;
    caps.qk_prologue = 0;   // no key workspace here
    bool on[4];
    if ((rc = validate_block(caps, io, dev.num_cus, on))) return rc;
    Plan plans[4];
    plan_block(caps, io, on, dev.num_cus, plans);
    // The scratch holds exactly the regions this call uses: TAIL then V2A.
    Workspace ws = {};
    for (int k = 0; k < 4; ++k)
        if (on[k] && plans[k].region != REGION_NONE) ws.rows[plans[k].region] = plans[k].ws_rows;
    const int64_t rows = ws.rows[REGION_TAIL] + ws.rows[REGION_V2A];
    if (rows * (cfg->head_dim + 2) * (int64_t)sizeof(float) > SCRATCH_BYTES) return LTXATTN_ERR_SCRATCH;
    ws.o = dev.scratch;
    ws.ml = dev.scratch + rows * cfg->head_dim;
    for (int n = 0; n < 4; ++n) {
        const int k = KIND_ORDER[n];
        if (!on[k]) continue;
        if ((rc = launch_plan(nullptr, cfg->head_dim, plans[k], ws, (hipStream_t)hip_stream, nullptr, nullptr)))
            return rc;
    }
    return LTXATTN_OK;
}

int ltxattn_profile_begin(ltxattn_handle *h, int32_t max_calls) {
    return ltxattn_profile_begin_kinds(h, max_calls, 0xFu);
}

int ltxattn_profile_begin_kinds(ltxattn_handle *h, int32_t max_calls, uint32_t kind_mask) {
    if (!h || max_calls < 1 || kind_mask == 0 || kind_mask > 0xFu) return LTXATTN_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return hip_fail(h, g.err);
    if (h->events) ltxattn_profile_end(h);
    h->events = (hipEvent_t *)calloc((size_t)max_calls * PROF_EVENTS, sizeof(hipEvent_t));
    h->prof_calls = (ltxattn_handle::ProfCall *)calloc((size_t)max_calls, sizeof(ltxattn_handle::ProfCall));
    if (!h->events || !h->prof_calls) {
        free(h->events);
        free(h->prof_calls);
        h->events = nullptr;
        h->prof_calls = nullptr;
        return LTXATTN_ERR_OOM;
    }
    for (int64_t i = 0; i < (int64_t)max_calls * PROF_EVENTS; ++i) {
        hipError_t e = hipEventCreate(&h->events[i]);
        if (e != hipSuccess) {
            for (int64_t j = 0; j < i; ++j) (void)hipEventDestroy(h->events[j]);
            free(h->events);
            free(h->prof_calls);
            h->events = nullptr;
            h->prof_calls = nullptr;
            return hip_fail(h, e);
        }
    }
    h->prof_max = max_calls;
    h->prof_n = 0;
    h->prof_kinds = kind_mask;
    return LTXATTN_OK;
}

int ltxattn_profile_read(ltxattn_handle *h, float *ms, int32_t max_calls, int32_t *n_calls) {
    if (!h || !ms || !n_calls || max_calls < 1 || !h->events) return LTXATTN_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    if (g.err != hipSuccess) return hip_fail(h, g.err);
    const int n = h->prof_n < max_calls ? h->prof_n : max_calls;
    for (int c = 0; c < n; ++c) {
        hipEvent_t *ev = h->events + (int64_t)c * PROF_EVENTS;
        const ltxattn_handle::ProfCall &pc = h->prof_calls[c];
        float *out = ms + (int64_t)c * LTXATTN_PROFILE_FLOATS;
        for (int i = 0; i < LTXATTN_PROFILE_FLOATS; ++i) out[i] = NAN;
        if (pc.sync < 0) continue;                          // no recorded kind ran
        hipError_t e = hipEventSynchronize(ev[pc.sync]);   // the call's last recorded event
        if (e != hipSuccess) return hip_fail(h, e);
        for (int k = 0; k < 4; ++k) {
            float tot = 0.f, ker = 0.f;
            if (pc.start[k] < 0) continue;                  // not recorded: NaN
            if (pc.end[k] != pc.start[k]) {   // else skipped: 0
                if ((e = hipEventElapsedTime(&tot, ev[pc.start[k]], ev[pc.end[k]])) != hipSuccess) return hip_fail(h, e);
                if ((e = hipEventElapsedTime(&ker, ev[pc.start[k]], ev[pc.mid[k] >= 0 ? pc.mid[k] : pc.end[k]]))
                    != hipSuccess)
                    return hip_fail(h, e);
            }
            out[k] = tot;
            out[5 + k] = ker;
        }
        if (pc.first >= 0) {
            float tot = 0.f;
            if ((e = hipEventElapsedTime(&tot, ev[pc.first], ev[pc.last])) != hipSuccess) return hip_fail(h, e);
            out[4] = tot;
        }
    }
    *n_calls = n;
    return LTXATTN_OK;
}

int ltxattn_profile_end(ltxattn_handle *h) {
    if (!h) return LTXATTN_ERR_INVALID_ARG;
    if (!h->events) return LTXATTN_OK;
    DeviceGuard g(h->device);
    for (int64_t i = 0; i < (int64_t)h->prof_max * PROF_EVENTS; ++i) (void)hipEventDestroy(h->events[i]);
    free(h->events);
    free(h->prof_calls);
    h->events = nullptr;
    h->prof_calls = nullptr;
    h->prof_max = h->prof_n = 0;
    return LTXATTN_OK;
}

}  // extern "C"

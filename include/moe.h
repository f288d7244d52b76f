/*
 * moe.h - C ABI of the fused FP8 x FP4 top-k Mixture-of-Experts layer for one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (pages: "MegaMoE" study notes, section "Dispatch阶段" and its flow
 * chart; "MonoMoe kernel — design" §1):
 *   route      top-k of softmax or sigmoid scores over E experts, optional
 *              renormalisation of the k weights
 *   bucketize  counting sort of the T*k (token, slot) pairs into per-expert
 *              contiguous segments: count, prefix sum, scatter of t*k + j
 *              ("05.10 Counting Sort / Bucketization", sections 2.1-2.3)
 *   quant      x BF16 -> FP8 E4M3 + one UE8M0 scale per 32 hidden elements
 *   GEMM1      per expert: rows x [W1; W3]^T, FP4 E2M1 weights with one UE8M0
 *              scale per 32 along K, FP32 accumulation; epilogue
 *              h = silu(gate) * up * topk_weight re-quantised to FP8 + UE8M0
 *   GEMM2      per expert: h x W2^T (FP4), FP32 accumulation -> BF16 rows
 *   combine    y[t] = BF16(sum over the token's k rows in FP32, slot order)
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never allocates, frees or keeps them.  Work is enqueued on the
 *     given HIP stream; no call but moe_check_status synchronises with the
 *     host.  Results are valid once the stream has reached the call.
 *   - Return 0 on success or a negative MOE_E* code.  Argument errors are
 *     detected on the host before anything is enqueued.  A kernel launch error
 *     returns MOE_EHIP; moe_error_string(MOE_EHIP) then holds the HIP message
 *     of the calling thread's last failure.
 *   - BF16 tensors are passed as uint16_t bit patterns, FP8/FP4 codes and
 *     UE8M0 scales as uint8_t.  All arrays are dense and row-major.
 *   - FP4 packing: element 2i of a row in the low nibble of byte i, element
 *     2i+1 in the high nibble.  Scales: one byte per 32 consecutive elements
 *     of a row, value 2^(b - 127).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)        /* bad pointer, size or shape */
#define MOE_EUNSUPPORTED (-2)  /* shape outside what the kernels handle */
#define MOE_EWORKSPACE (-3)    /* workspace too small or misaligned */
#define MOE_EHIP (-4)          /* HIP runtime / launch failure */
#define MOE_ETIMEOUT (-5)      /* moe_check_status: a bounded wait inside the last call gave up */
#define MOE_ESCRATCH (-6)      /* moe_route_noalloc: T * topk above its static scratch's limit */

#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1

/* Layer shape.
 *   T         tokens (>= 0; T == 0 is a no-op)
 *   H         hidden size, multiple of 128
 *   I         intermediate size of one projection (gate or up), multiple of 128
 *   E         experts, 1..1024
 *   topk      experts per token, 1..min(E, 16)
 *   score_fn  MOE_SCORE_SOFTMAX or MOE_SCORE_SIGMOID (routing inside the library)
 *   renorm    nonzero: the k weights are divided by their sum
 * T <= 2^24 and T*H, T*topk*I and H*I each below 2^32 (MOE_EUNSUPPORTED
 * otherwise): the GEMMs address activation rows and one expert's weights with
 * 32-bit byte offsets. */
typedef struct moe_dims {
    int64_t T;
    int32_t H;
    int32_t I;
    int32_t E;
    int32_t topk;
    int32_t score_fn;
    int32_t renorm;
} moe_dims_t;

/* Flags of moe_forward.  The GEMMs run either as tiled kernels (128 x 512
 * output tiles staged through LDS, for many rows per expert) or as narrow
 * kernels (weights streamed from HBM straight into registers over many small
 * workgroups, for few rows per expert, the decode regime).  By default
 * moe_forward takes the narrow kernels when T * topk <= 3 * E, else the tiled
 * GEMM1 and GEMM2 as two launches ordered by the stream.  MOE_FLAG_ONE_LAUNCH
 * runs the tiled GEMM1 -> SwiGLU -> GEMM2 as one persistent launch whose GEMM2
 * tiles wait on per-m-tile ready counters, experts grouped in waves ("MegaMoE"
 * notes, "Scheduler" and "Wave"); on one MI355X it measured slower than the
 * two launches at the DeepSeek-V3-like and 256-expert shapes, so it is not
 * the default.  MOE_FLAG_ONE_KERNEL runs the whole layer (routing, bucketing,
 * quantisation, the narrow GEMMs and the combine) as one cooperative launch
 * whose phases hand over by arrival counts ("MonoMoe kernel — design" §1;
 * "MegaMoE：把通信和计算融合到一个 Mega Kernel", arrival-count polling); it
 * needs T * topk <= 1024 (else MOE_EUNSUPPORTED) and implies the narrow GEMMs.
 * On one MI355X its waits cost more than the launch boundaries they replace
 * (84 against 44 us at the decode shape), so it is not the default either.  MOE_FLAG_NARROW | MOE_FLAG_ONE_LAUNCH runs the narrow GEMM1
 * -> SwiGLU -> GEMM2 as one launch whose GEMM2 units wait on per-sub-tile
 * ready counters; measured slower than the two narrow launches at the decode
 * shape (GEMM2 cannot start before the slowest GEMM1 unit of its rows), so it
 * is opt-in.  All paths meet the same tolerance against the definition.
 * NARROW together with TILED is MOE_EINVAL, and so is ONE_KERNEL together with
 * TILED or ONE_LAUNCH. */
#define MOE_FLAG_NONE 0u
#define MOE_FLAG_NARROW 1u
#define MOE_FLAG_TILED 2u
#define MOE_FLAG_ONE_LAUNCH 4u
#define MOE_FLAG_ONE_KERNEL 8u
/* Weight-layout and debugging flags ("MegaMoE：把通信和计算融合到一个 Mega Kernel",
 * Python API walk-through: the caller transforms the weights once, then makes
 * one call per batch; "MonoMoe kernel — design" §2-§3 for bounded waits):
 *   W13_PREINTERLEAVED  w13 (codes and scales) is in the pages' gate/up row
 *                       interleave with granularity 8 ("MegaMoE" study notes,
 *                       "原始权重布局"): rows [16 i, 16 i + 8) are gate rows
 *                       [8 i, 8 i + 8) and rows [16 i + 8, 16 i + 16) the up
 *                       rows of the same 8 columns.  Without it, rows [0, I)
 *                       are gate and [I, 2I) up.  Results are bit-identical.
 *   W_SCALES_PER_ROW    w13_sf and w2_sf are per-row [E, rows, K/32] (as
 *                       moe_pack_weights writes them) instead of K-step major
 *                       [E, K/128, rows, 4].  Results are bit-identical; the
 *                       per-row layout costs one load per scale row and K step
 *                       instead of one per 64 rows.
 *   KEEP_INTERMEDIATES  accepted for callers that state it: every call leaves
 *                       its intermediates in the workspace at the offsets
 *                       moe_workspace_layout reports, until the next call.
 *   DEBUG_SPIN_BOUND    the ready-counter waits of the one-launch GEMM paths
 *                       give up after one failed poll instead of about 0.5 s
 *                       of polling; a wait that gives up sets the status word
 *                       (moe_check_status reports MOE_ETIMEOUT) and the output
 *                       is then invalid.  For exercising the failure report;
 *                       MOE_EINVAL together with ONE_KERNEL, whose routing
 *                       hand-off guards the tables the later phases index
 *                       with (giving up there early could read stale
 *                       indices). */
#define MOE_FLAG_W13_PREINTERLEAVED 16u
#define MOE_FLAG_W_SCALES_PER_ROW 32u
#define MOE_FLAG_KEEP_INTERMEDIATES 64u
#define MOE_FLAG_DEBUG_SPIN_BOUND 128u
/* Block-FP8 weights ("MonoMoe kernel — design", the fixed-shape paragraph:
 * block-FP8 128 x 128 weights, for the decode shape of at most 8 tokens): w13
 * and w2 hold E4M3 codes [E, 2I, H] and [E, H, I], w13_sf and w2_sf one float32
 * scale per 128 x 128 block, [E, 2I/128, H/128] and [E, H/128, I/128]
 * (moe_pack_weights_fp8_block128 writes both).  x and h are quantised to E4M3
 * with one float32 scale per row per 128 elements (scale = max|v| / 448).  The
 * GEMMs run as the narrow kernels in two launches, with a quantisation launch
 * for h between them (a 128-column group spans several workgroups' units).
 * MOE_EUNSUPPORTED with TILED, ONE_LAUNCH or ONE_KERNEL; MOE_EINVAL with
 * W13_PREINTERLEAVED or W_SCALES_PER_ROW. */
#define MOE_FLAG_WEIGHTS_FP8_BLOCK128 256u
/* Staged FP4 weight codes ("MegaMoE：把通信和计算融合到一个 Mega Kernel", Python API
 * walk-through: a one-time transform of the weights before the per-batch
 * calls): w13 and w2 hold the codes as moe_stage_weights writes them; the
 * scales keep the layout the other flags select.  Results are bit-identical to
 * the canonical layout's.  MOE_EINVAL with W13_PREINTERLEAVED (the staged
 * layout is made from the canonical one) or WEIGHTS_FP8_BLOCK128. */
#define MOE_FLAG_W_STAGED 512u

#define MOE_NUM_STAGE_EVENTS 5

/* Arguments of moe_forward.
 *   x         device, BF16 [T, H]
 *   logits    device, float32 [T, E] router logits; or NULL, and then
 *   topk_idx  device, int32 [T, topk] expert ids (entries < 0 are skipped) and
 *   topk_w    device, float32 [T, topk] routing weights
 *   w13       device, FP4 [E, 2I, H/2]: rows [0, I) gate (W1), [I, 2I) up (W3);
 *             the staged layout (moe_stage_weights) with MOE_FLAG_W_STAGED, as w2
 *   w13_sf    device, UE8M0 [E, H/128, 2I, 4]: K-step major (moe_scales_kmajor
 *             of the per-row [E, 2I, H/32] scales); per-row [E, 2I, H/32]
 *             with MOE_FLAG_W_SCALES_PER_ROW
 *   w2        device, FP4 [E, H, I/2]
 *   w2_sf     device, UE8M0 [E, I/128, H, 4]: K-step major; per-row
 *             [E, H, I/32] with MOE_FLAG_W_SCALES_PER_ROW
 *   y         device, BF16 [T, H], written
 *   ws        device workspace of at least moe_workspace_size() bytes,
 *             256-byte aligned, zeroed once by moe_workspace_init() after it is
 *             allocated; every call leaves it ready for the next call.  One
 *             workspace must not be used by two calls that may overlap.
 *   stage_events  NULL, or MOE_NUM_STAGE_EVENTS caller-created HIP events that
 *             are recorded on s before routing, before GEMM1, before GEMM2,
 *             before the combine and after it (for per-stage timing); with
 *             MOE_FLAG_ONE_LAUNCH the third is recorded after that launch,
 *             right before the fourth; with MOE_FLAG_ONE_KERNEL the second,
 *             third and fourth are recorded after the one launch.
 *   kernel_events  NULL, or 2 caller-created HIP events that the GEMM1 launch
 *             itself carries (hipExtLaunchKernel): they take the time the
 *             GEMM1 kernel starts and the time it ends, so their elapsed time
 *             is the kernel's duration without launch gaps (for rooflines).
 *             With MOE_FLAG_ONE_LAUNCH they bracket the fused GEMM launch;
 *             MOE_FLAG_ONE_KERNEL does not use them. */
typedef struct moe_args {
    moe_dims_t dims;
    const uint16_t* x;
    const float* logits;
    const int32_t* topk_idx;
    const float* topk_w;
    const uint8_t* w13;
    const uint8_t* w13_sf;
    const uint8_t* w2;
    const uint8_t* w2_sf;
    uint16_t* y;
    void* ws;
    size_t ws_bytes;
    uint32_t flags;
    hipEvent_t* stage_events;
    hipEvent_t* kernel_events;
} moe_args_t;

/* Byte offsets of the intermediates inside the workspace after moe_forward
 * (for inspection and tests).  Positions p are slot positions: expert e owns
 * p in [offsets[e], offsets[e+1]).
 *   topk_idx  int32 [T, topk]     routing result used (copy of the input ids
 *                                 when the caller routed)
 *   topk_w    float32 [T, topk]
 *   counts    int32 [E]
 *   offsets   int32 [E + 1]       exclusive prefix sum of counts
 *   slot_src  int32 [T*topk]      t*topk + j of position p (first offsets[E] valid)
 *   slot_of   int32 [T, topk]     position of pair (t, j), -1 when skipped
 *   xq, xsf   uint8 [T, H], [H/128, T, 4]        quantised x (scales K-step major;
 *                                               float32 [H/128, T] with block-FP8 weights)
 *   hq, hsf   uint8 [T*topk, I], [I/128, T*topk, 4]  quantised h by position (float32
 *                                               [I/128, T*topk] with block-FP8 weights)
 *   o         BF16 [T*topk, H]                  GEMM2 rows by position
 *   status    int32 [1]   nonzero if a wait of the one-launch GEMMs gave up in
 *                         the last call (its output is then invalid); every
 *                         call clears it before its GEMMs */
typedef struct moe_layout {
    size_t topk_idx, topk_w, counts, offsets, slot_src, slot_of;
    size_t xq, xsf, hq, hsf, o;
    size_t status;
    size_t total;
} moe_layout_t;

/* Size in bytes of the caller-owned workspace moe_forward and moe_route need
 * for d ("MonoMoe kernel — design" §4: the host sizes the scratchpad from the
 * library, which exports its size; "MegaMoE" study notes, "WorkSpace").
 *   d      host pointer to the shape (checked as for moe_forward)
 *   bytes  host pointer, out
 * Returns MOE_EINVAL / MOE_EUNSUPPORTED for a bad shape, else MOE_OK. */
int moe_workspace_size(const moe_dims_t* d, size_t* bytes);

/* Offsets of the intermediates in the workspace for d (the same pages as
 * moe_workspace_size).  d and out are host pointers; errors as for
 * moe_workspace_size. */
int moe_workspace_layout(const moe_dims_t* d, moe_layout_t* out);

/* Zero a freshly allocated workspace (enqueued on s).  Needed once per
 * allocation: the library's internal counters must start at zero, and each
 * call resets them before it returns ("MonoMoe kernel — design" §4 keys the
 * same one-time zeroing on the buffer's identity). */
int moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t s);

/* Top-k routing and counting-sort bucketisation ("MonoMoe kernel — design" §1
 * phase 1; "05.10 Counting Sort / Bucketization" sections 2.1-2.3).
 *   logits    device float32 [T, E]
 *   topk_idx  device int32 [T, topk] out: chosen experts, decreasing logit,
 *             equal logits by increasing expert id
 *   topk_w    device float32 [T, topk] out: weights (see moe_dims_t)
 *   counts    device int32 [E] out
 *   offsets   device int32 [E + 1] out: exclusive prefix sum of counts
 *   slot_src  device int32 [T*topk] out: t*topk + j for each position; the
 *             order inside an expert's segment is unspecified
 *   slot_of   device int32 [T, topk] out: position of (t, j)
 *   ws        workspace as for moe_forward */
int moe_route(const moe_dims_t* d, const float* logits, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* slot_src, int32_t* slot_of,
              void* ws, size_t ws_bytes, hipStream_t s);

/* moe_route without a workspace, for callers that cannot allocate device memory
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * moe_route, minus ws and ws_bytes.  The routing counters and tables live in a
 * static device array of the library (about 2.4 MiB per device, held until the
 * process ends), sized for T * topk <= 262144 routed pairs with any E <= 1024;
 * a larger call returns MOE_ESCRATCH before anything is enqueued.  The call
 * allocates nothing: it enqueues a small fill kernel that zeroes the array's
 * counters, then the routing kernels.  Every call on one device shares that
 * device's array, so two calls that may overlap on one device (different
 * streams, or one stream while another call is in flight elsewhere) race and
 * must be ordered by the caller. */
int moe_route_noalloc(const moe_dims_t* d, const float* logits, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* slot_src, int32_t* slot_of,
                      hipStream_t s);

/* Per-row activation quantisation ("MegaMoE" notes, "Dispatch阶段"): each group
 * of 32 consecutive elements of a row gets the smallest power-of-two scale s
 * with max|v| <= 448 s, and codes v/s rounded to nearest-even E4M3.
 *   x   device BF16 [rows, cols]; cols a multiple of 32
 *   q   device uint8 [rows, cols] out: E4M3 codes
 *   sf  device uint8 [rows, cols/32] out: UE8M0 scale bytes */
int moe_quant_act(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, uint8_t* sf,
                  hipStream_t s);

/* Weight quantisation ("MegaMoE" notes, "Expert矩阵权重量化"): BF16 [rows, cols]
 * to FP4 E2M1 with one UE8M0 scale per 32 consecutive elements of a row
 * (smallest power of two s with max|v| <= 6 s; nearest-even codes).
 *   w   device BF16 [rows, cols]; cols a multiple of 32
 *   q   device uint8 [rows, cols/2] out: packed E2M1
 *   sf  device uint8 [rows, cols/32] out */
int moe_pack_weights(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* q, uint8_t* sf,
                     hipStream_t s);

/* Block-FP8 weight quantisation ("MonoMoe kernel — design", fixed-shape
 * paragraph): BF16 [rows, cols] to E4M3 codes with one float32 scale per
 * 128 x 128 block: s = max|v| / 448 over the block (1 for an all-zero block),
 * codes nearest-even E4M3 of v / s.  A stack of matrices [E, N, K] is one
 * [E * N, K] call when N is a multiple of 128.
 *   w    device BF16 [rows, cols]; rows and cols multiples of 128
 *   q    device uint8 [rows, cols] out
 *   sf   device float32 [rows/128, cols/128] out
 * MOE_EINVAL for bad sizes or pointers (w 16-byte, q 16-byte, sf 4-byte aligned). */
int moe_pack_weights_fp8_block128(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* q, float* sf,
                                  hipStream_t s);

/* Weight-scale layout change for moe_forward (the layer's counterpart of a
 * one-time weight transform): per-row scales [mats, rows, cols/32] become K-step
 * major [mats, cols/128, rows, 4], so that the scales of many rows for one
 * 128-wide K step are contiguous (one load per row block instead of one per
 * row).
 *   sf    device uint8 [mats, rows, cols/32] (e.g. from moe_pack_weights)
 *   cols  K, a multiple of 128
 *   out   device uint8 [mats, cols/128, rows, 4]; must not overlap sf */
int moe_scales_kmajor(const uint8_t* sf, int64_t mats, int32_t rows, int32_t cols, uint8_t* out,
                      hipStream_t s);

/* Weight-code layout change for moe_forward with MOE_FLAG_W_STAGED (a
 * one-time weight transform, as the scale layout change above; "MegaMoE" study
 * notes, "原始权重布局", for the canonical gate-then-up row order it starts
 * from).  Each matrix's packed codes are regrouped so that the GEMMs' weight
 * loads read whole contiguous KiB: rows in groups of 16, and the 64 bytes of K
 * step ks (128 values) of row c of group g at byte (g * cols/128 + ks) * 1024 +
 * 64 c of the matrix.  Group g = 8 b + n holds
 *   W13 (is_w13 != 0, rows = 2I): projection n & 1 (0 gate, 1 up) of I column
 *       64 b + 4 c + n / 2, i.e. canonical row (n & 1) * I + 64 b + 4 c + n / 2;
 *   W2  (is_w13 == 0, rows = H):  canonical row 128 b + 8 c + n.
 *   w     device uint8 [mats, rows, cols/2], canonical row order (moe_pack_weights)
 *   rows  2I (W13) or H (W2), a multiple of 128
 *   cols  K (H for W13, I for W2), a multiple of 128
 *   out   device uint8, mats * rows * cols/2 bytes; must not overlap w
 * MOE_EINVAL for bad sizes or pointers (w and out 16-byte aligned). */
int moe_stage_weights(const uint8_t* w, int64_t mats, int32_t rows, int32_t cols, int32_t is_w13, uint8_t* out,
                      hipStream_t s);

/* The whole layer ("MegaMoE" study notes, "Dispatch阶段" flow chart: route or
 * take topk_idx/topk_w, counting-sort bucketisation, quantise x, GEMM1 +
 * SwiGLU*weight -> FP8, GEMM2 -> BF16, combine into y; "MegaMoE：把通信和计算
 * 融合到一个 Mega Kernel", Python API walk-through: one call per batch on a
 * caller-allocated workspace and transformed weights).
 *   a  host pointer to the arguments (moe_args_t above); every tensor in it is
 *      device memory owned by the caller.
 * Returns MOE_EINVAL for a NULL or misaligned pointer (x, w13, w2, y 16-byte
 * aligned; scales 4-byte aligned), an unknown or contradictory flag set;
 * MOE_EUNSUPPORTED for a shape outside moe_dims_t's limits; MOE_EWORKSPACE
 * for a workspace below moe_workspace_size or not 256-byte aligned; MOE_EHIP
 * for a launch failure.  T == 0 returns MOE_OK without launching. */
int moe_forward(const moe_args_t* a, hipStream_t s);

/* Status of the last call on workspace ws ("MonoMoe kernel — design" §2-§3:
 * waits are bounded so a broken hand-off ends instead of hanging).
 * Synchronises stream s (waits for every call enqueued on it), then reads the
 * status word at its fixed offset in the workspace header (the same for every
 * shape).  Returns MOE_OK, or MOE_ETIMEOUT when a bounded wait of the last
 * moe_forward on ws gave up (its output is then invalid; never in a correct
 * run without MOE_FLAG_DEBUG_SPIN_BOUND), or MOE_EINVAL for a NULL or
 * misaligned ws, or MOE_EHIP. */
int moe_check_status(const void* ws, hipStream_t s);

/* Measurement helper: read `bytes` from src once with 16-byte loads spread over
 * the GPU and nothing else to do (the HBM read ceiling of a footprint, the
 * yardstick beside the roofline of a weight-streaming kernel).
 *   src    device, 16-byte aligned; bytes a multiple of 16
 *   sink   device uint32, left unchanged by real data (a store on one value
 *          keeps the loads from being optimised away)
 *   start, stop  NULL, or caller-created events the launch carries
 *          (hipExtLaunchKernel): they take the kernel's start and end times
 * MOE_EINVAL for bad pointers or sizes; bytes == 0 launches nothing (the
 * events are then recorded on s). */
int moe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipEvent_t start, hipEvent_t stop,
                    hipStream_t s);

/* Static text for a return code (for MOE_EHIP: the calling thread's last HIP
 * error message). */
const char* moe_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */

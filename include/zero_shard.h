/*
 * zero_shard.h -- C ABI of the ZeRO-1/2 owner-shard step on MI355X (gfx950).
 *
 * The owner-shard step is the part of a ZeRO-1/2 data-parallel step that the
 * owner of one partition of a flat parameter group runs after the backward
 * pass:
 *
 *   1. layout   the group's tensors are flattened into one buffer, padded for
 *               alignment and cut into N equal partitions, one per rank
 *               (ZeRO-2 source walkthrough, discosf.com, sections 2.1 and 4.1);
 *   2. reduce   the owner receives the sum of the N ranks' 16-bit gradients
 *               for its partition (ZeRO 优化器, cookllm.com, "ZeRO Stage 1"
 *               gradient sync; ZeRO-2 source walkthrough sections 4.2 and 三);
 *   3. check    unscale by the loss scale, test for inf/NaN (an overflow skips
 *               the step) and take the squared L2 norm for clipping (wmrh.cn
 *               ZeRO article, section 3.1 fp16 block and section 3.3
 *               gradient_clipping);
 *   4. adamw    AdamW on the partition's fp32 master weights, m and v, then the
 *               16-bit copy of the new weights (ZeRO-2 source walkthrough,
 *               sections 4.1 step 3 and 4.3);
 *   5. scaler   dynamic loss-scale update (wmrh.cn article, section 3.1), on the
 *               host (zero_loss_scaler_update) or on the device
 *               (zero_step_control_update, with the *_ctl variants of 3 and 4
 *               reading their per-step scalars from device memory so that a
 *               step can be captured once in a HIP graph and replayed).
 *
 * Conventions for every call:
 *   - Buffers are flat arrays.  "device" pointers are HIP device memory owned
 *     by the caller; "host" pointers are ordinary host memory owned by the
 *     caller.  The library never allocates, frees or keeps a pointer after a
 *     call returns, and keeps no state between calls, with one exception:
 *     zero_reduce_check_owned_noalloc uses a scratch array of the library's
 *     own, one per device, and remembers its device address.
 *   - 16-bit data (gradients, the parameter copy) is passed as raw 16-bit
 *     patterns; `dtype` says whether they are IEEE binary16 or bfloat16.
 *   - Device calls are asynchronous and ordered on `stream` (0 = the null
 *     stream).  None of them synchronises.  Any element offset is accepted;
 *     pointers that share their alignment modulo 16 bytes take the 128-bit
 *     vector path for everything but at most 7 leading and 7 trailing elements.
 *   - Element counts are limited by memory only: a pass over more elements
 *     than one launch's 32-bit grid holds (about 34e9) is issued as several
 *     launches, in order, on the same stream.
 *   - Arguments are checked before anything is launched; a bad argument
 *     returns ZERO_EINVAL (or ZERO_ERANGE for sizes that overflow) and
 *     launches nothing.  A failed launch returns ZERO_EDEVICE.  No call
 *     aborts, throws or prints.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum zero_status {
    ZERO_OK = 0,
    ZERO_EINVAL = -1,  /* bad argument: null pointer, negative size, unknown dtype ... */
    ZERO_ERANGE = -2,  /* a size or offset overflows int64                              */
    ZERO_EDEVICE = -3  /* a HIP launch failed                                           */
};

enum zero_dtype {
    ZERO_FP16 = 1,     /* IEEE 754 binary16 */
    ZERO_BF16 = 2      /* bfloat16          */
};

#define ZERO_MAX_RANKS 16

/* Result of the check phase.  Lives in device memory; written by
 * zero_unscale_check_norm, read by zero_adamw_step on the device, and copied
 * to the host by the caller only for the loss-scale update.  16 bytes. */
typedef struct zero_step_result {
    double sumsq;        /* sum over the checked elements of (value * inv_scale)^2, fp64;
                            value * inv_scale is the fp32 product                       */
    uint32_t overflow;   /* 1 if some checked element is +-inf or NaN, else 0          */
    float inv_scale;     /* the unscale factor the check used                           */
} zero_step_result;

/* AdamW hyper-parameters (wmrh.cn article section 3.1 ds_config: betas,
 * eps, weight_decay; learning rate per the run).  `step` is t counted from 1,
 * i.e. the value after this step's increment.  max_grad_norm <= 0 turns
 * clipping off. */
typedef struct zero_adamw_hparams {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
    int64_t step;
} zero_adamw_hparams;

/* Dynamic loss-scale state (host).  wmrh.cn article section 3.1 fp16 block:
 * loss_scale 0 (dynamic), loss_scale_window 1000, min_loss_scale 1. */
typedef struct zero_loss_scaler {
    double scale;       /* current loss scale S (a power of two)          */
    double min_scale;   /* S never drops below this                       */
    int64_t window;     /* clean steps in a row before S doubles          */
    int64_t clean;      /* clean steps since the last change              */
    int64_t skipped;    /* total steps skipped for overflow               */
} zero_loss_scaler;

/* Device-resident step control: the dynamic loss scaler of zero_loss_scaler
 * and the AdamW step count, kept in device memory and advanced on the device
 * (zero_step_control_update), so that a loop of owner steps needs no host
 * round trip -- for example one step captured in a HIP graph and replayed.
 * Filled on the host by zero_step_control_init, copied to the device by the
 * caller, then only read by the *_ctl calls and advanced by
 * zero_step_control_update.  The rules are those of zero_loss_scaler_update
 * and zero_adamw_step (wmrh.cn article section 3.1: dynamic loss scaling,
 * AdamW betas).  72 bytes, 8-byte aligned. */
typedef struct zero_step_control {
    double scale;       /* loss scale S of the next step                        */
    double min_scale;   /* S never drops below this                             */
    int64_t window;     /* clean steps in a row before S doubles                */
    int64_t clean;      /* clean steps since the last change                    */
    int64_t skipped;    /* steps skipped for overflow                           */
    int64_t t;          /* AdamW steps applied so far                           */
    float divisor;      /* D: gradients are unscaled by 1 / (S * D)             */
    float inv_scale;    /* fp32(1 / (S * D)), the next step's unscale factor    */
    float beta1, beta2; /* AdamW betas                                          */
    float bc1, bc2;     /* fp32(1 - beta1^(t+1)), fp32(1 - beta2^(t+1)): the
                           next applied step's bias corrections                 */
} zero_step_control;

/* One tensor of a flattened group (device array of these in flat order, for
 * zero_flat_gather / zero_flat_scatter).  32 bytes. */
typedef struct zero_tensor_desc {
    void* ptr;          /* device pointer to the tensor's `numel` 16-bit values   */
    int64_t offset;     /* index of the tensor's first element in the flat buffer */
    int64_t numel;      /* elements                                               */
    int64_t reserved;   /* set to 0                                               */
} zero_tensor_desc;

/* A range of elements [offset, offset + count) of the flat buffers a call is
 * given (for the *_ranges calls).  16 bytes. */
typedef struct zero_range {
    int64_t offset;     /* first element, >= 0  */
    int64_t count;      /* elements, >= 0       */
} zero_range;

/* ---------------------------------------------------------------- host ---- */

/* Flatten + align + partition (ZeRO-2 source walkthrough, section 4.1 steps
 * 1-2; section 2.1 "near-equal partitions").  Tensors are laid back to back in
 * the given order: tensor_offsets[k] = numels[0] + ... + numels[k-1].  The
 * total Phi is padded at the tail to the next multiple of world*align_elems
 * (the pages use align_elems = 2, i.e. 4 bytes of 16-bit data); partition p
 * is [part_begin[p], part_begin[p+1]) with part_begin[p] = p * padded/world.
 *   numels[n_tensors]          host, in     element counts, each >= 0
 *   tensor_offsets[n_tensors]  host, out    (may be NULL when n_tensors == 0)
 *   part_begin[world + 1]      host, out
 *   padded_total               host, out
 * Errors: ZERO_EINVAL for world < 1, align_elems < 1, a negative count or a
 * NULL output; ZERO_ERANGE if the padded total overflows int64. */
int zero_partition_layout(const int64_t* numels, int64_t n_tensors, int32_t world,
                          int32_t align_elems, int64_t* tensor_offsets, int64_t* part_begin,
                          int64_t* padded_total);

/* Reduce-bucket windows (ZeRO-2 source walkthrough, section 4.2: gradients are
 * gathered into buckets of reduce_bucket_size elements and each full bucket
 * is reduced).  Tensors are taken in order; a bucket that cannot take the
 * next whole tensor is closed; an empty bucket takes any tensor, however large.
 *   bucket_first[n_tensors + 1]  host, out  first tensor of each bucket, then n_tensors
 *   n_buckets                    host, out
 * Errors: ZERO_EINVAL for bucket_cap < 1, a negative count or a NULL output. */
int zero_bucket_layout(const int64_t* numels, int64_t n_tensors, int64_t bucket_cap,
                       int64_t* bucket_first, int64_t* n_buckets);

/* Model-state bytes per rank under ZeRO stage 0..3 (ZeRO 优化器 memory tables;
 * ZeRO / DeepSpeed 深度解读报告 section 3.3): 2 B of 16-bit parameters, 2 B of
 * 16-bit gradients and 12 B of fp32 master + m + v per element; stage >= 1
 * shards the 12 B, stage >= 2 the gradients, stage 3 the parameters.  A
 * sharded part holds P = padded_total / world elements; unsharded parts hold
 * numel_total.  With padded_total == numel_total this is 16*Phi,
 * 4*Phi + 12*Phi/N, 2*Phi + 14*Phi/N and 16*Phi/N.
 * Errors: ZERO_EINVAL for stage outside 0..3, world < 1, padded_total <
 * numel_total or not a multiple of world; ZERO_ERANGE on overflow. */
int zero_memory_bytes(int32_t stage, int64_t numel_total, int64_t padded_total, int32_t world,
                      int64_t* bytes_out);

/* Dynamic loss-scale update after a step (wmrh.cn article section 3.1).  On
 * overflow: S = max(S/2, min_scale), clean = 0, skipped += 1.  Otherwise
 * clean += 1 and, when clean reaches window, S = 2S and clean = 0.
 * Errors: ZERO_EINVAL for a NULL state or window < 1. */
int zero_loss_scaler_update(zero_loss_scaler* scaler, uint32_t overflow);

/* Initial device step control (host struct, to be copied to device memory):
 * S = scale0, t = 0, no clean or skipped steps; inv_scale, bc1 and bc2 for
 * the first step (bc = 1 - beta, computed in fp64 and rounded once).
 * Errors: ZERO_EINVAL for a NULL output, scale0 or min_scale not finite and
 * > 0, window < 1, divisor not finite and > 0, or a beta outside [0, 1). */
int zero_step_control_init(zero_step_control* ctl, double scale0, double min_scale,
                           int64_t window, float divisor, float beta1, float beta2);

/* Text for a status code (static storage). */
const char* zero_status_str(int status);

/* -------------------------------------------------------------- device ---- */

/* fp32 master weights of a partition from its 16-bit copy: master[i] =
 * float(param16[i]), exact (ZeRO-2 source walkthrough, section 4.1 step 3:
 * each rank clones its 16-bit partition to fp32).
 *   master[count]   device, out (fp32)
 *   param16[count]  device, in  (16-bit patterns of `dtype`) */
int zero_init_master(float* master, const void* param16, int64_t count, int32_t dtype,
                     hipStream_t stream);

/* Bucket copy-in (ZeRO-2 source walkthrough section 2.4: with
 * contiguous_gradients each gradient is copied into one contiguous buffer;
 * section 4.2: each ready gradient goes into the reduce bucket at its place in
 * the flattened group):
 *   flat[d.offset + j] = d.ptr[j] for every descriptor d and j < d.numel;
 *   every flat element in [0, flat_count) that no descriptor covers is set to 0
 *   (the alignment padding).
 *   flat[flat_count]   device, out, 16-bit patterns (copied unchanged)
 *   descs[n_descs]     device array in flat order: descs[k+1].offset >=
 *                      descs[k].offset + descs[k].numel (a zero-size tensor
 *                      may share the offset of the tensor after it), every
 *                      range inside [0, flat_count); each ptr valid for numel
 *                      values.
 * The kernel reads a tensor only at indices below its numel and writes the
 * flat buffer only below flat_count, so a table that breaks the ordering rule
 * gives wrong values but no out-of-range access.
 * Errors: ZERO_EINVAL for flat_count < 0, n_descs < 0, or a NULL pointer with
 * a nonzero count. */
int zero_flat_gather(void* flat, int64_t flat_count, const zero_tensor_desc* descs,
                     int64_t n_descs, hipStream_t stream);

/* Write-back of an updated flat 16-bit buffer into its tensors (ZeRO-2 source
 * walkthrough section 4.4: after the step the updated partitions are gathered
 * back into the full parameters):  d.ptr[j] = flat[d.offset + j] for every
 * descriptor d and j < d.numel.  Arguments as for zero_flat_gather; flat is
 * read only. */
int zero_flat_scatter(const void* flat, int64_t flat_count, const zero_tensor_desc* descs,
                      int64_t n_descs, hipStream_t stream);

/* Reduce to the owner: dst[i] = round16(((0 + g_0[i]) + g_1[i]) + ... + g_{N-1}[i]),
 * the additions done in fp32 (each rounded to nearest-even) in rank order
 * starting from +0, and the result rounded once to the 16-bit type, ties to
 * even.  Starting from +0 makes a column of -0 values sum to +0.  An inf/NaN
 * input or a sum beyond the 16-bit range gives inf/NaN in dst, which the
 * check phase then flags.
 * (ZeRO 优化器 "ZeRO Stage 1": after the reduce the owner holds the sum of all
 * ranks' gradients; ZeRO-2 source walkthrough section 三: the reduced data is
 * fp16/bf16.)
 *   dst[count]       device, out
 *   srcs[n_ranks]    host array of device pointers, each to count 16-bit values
 *   n_ranks          1 .. ZERO_MAX_RANKS
 * dst may be the same pointer as one srcs[k] (in-place into the owner's own
 * buffer); no other overlap is allowed. */
int zero_reduce_owned(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count,
                      int32_t dtype, hipStream_t stream);

/* Reduce to the owner and check, fused: the same result as
 * zero_reduce_owned(dst, srcs, ...) followed by zero_unscale_check_norm(dst,
 * ...), in one pass that never re-reads dst (2 bytes per element less HBM
 * traffic).  Arguments as in those two calls.  Reduce windows of one step
 * (bucket x owner ranges) checked in turn on one stream form one global
 * result when every call after the first passes accumulate != 0. */
int zero_reduce_check_owned(void* dst, const void* const* srcs, int32_t n_ranks, int64_t count,
                            int32_t dtype, float inv_scale, zero_step_result* res,
                            void* workspace, size_t workspace_bytes, int32_t accumulate,
                            hipStream_t stream);

/* zero_reduce_check_owned without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the check partials live in a
 * scratch array inside the library, one per device, allocated when the
 * library's code is loaded on that device and held until the process ends
 * (25,178,368 bytes, the workspace of 2^32 elements).  The call itself
 * allocates nothing.  Same arguments and result as
 * zero_reduce_check_owned.
 *   count  at most 2^32 elements; a larger count returns ZERO_ERANGE and
 *          launches nothing
 * Every call on a device shares that device's scratch array: calls that can
 * overlap on one device (on different streams, or from several host threads
 * without ordering) race and give wrong results.  The array needs no
 * clearing: each call writes every partial it reads.  ZERO_EDEVICE if the
 * device of `stream` (the current device for the null stream) cannot be
 * queried. */
int zero_reduce_check_owned_noalloc(void* dst, const void* const* srcs, int32_t n_ranks,
                                    int64_t count, int32_t dtype, float inv_scale,
                                    zero_step_result* res, int32_t accumulate,
                                    hipStream_t stream);

/* Bytes of device workspace that zero_unscale_check_norm and
 * zero_reduce_check_owned need for `count` elements: one 12-byte partial per
 * 2048 elements plus the fold levels (about count / 170 bytes; 50.5 MB for
 * 8.62e9 elements, 16 bytes for count 0). */
size_t zero_check_workspace_bytes(int64_t count);

/* Unscale + overflow check + squared norm over grad16[0, count):
 *   overflow = some element is +-inf or NaN (exponent field all ones);
 *   sumsq    = sum of ((double)(value * inv_scale))^2, the product taken in
 *              fp32 and the squares accumulated in fp64 (each square is
 *              exact; the summation order is fixed for a given count and
 *              pointer alignment, so repeated calls give identical bits).
 * With accumulate == 0 the call overwrites *res; with accumulate != 0 it adds
 * its sumsq to res->sumsq and ORs its flag into res->overflow, so several
 * owner ranges checked in turn on one stream form one global result.
 * res->inv_scale is set to inv_scale either way.
 *   grad16[count]   device, in
 *   inv_scale       1 / (loss scale * divisor), finite and > 0 (ZERO_EINVAL
 *                   otherwise); a power of two makes the unscale exact
 *   res             device, out (in/out when accumulating)
 *   workspace       device scratch of at least zero_check_workspace_bytes(count)
 *                   bytes, 8-byte aligned; its contents are overwritten, need
 *                   no initialisation and must not be shared by calls that may
 *                   overlap. */
int zero_unscale_check_norm(const void* grad16, int64_t count, int32_t dtype, float inv_scale,
                            zero_step_result* res, void* workspace, size_t workspace_bytes,
                            int32_t accumulate, hipStream_t stream);

/* Fused AdamW over one partition (decoupled weight decay with bias-corrected
 * moments, eps added after the square root), reading the check result on the
 * device: if res->overflow is set the kernel writes nothing (the step is
 * skipped; the caller keeps t).  Otherwise, with
 *   coef = max_grad_norm / (sqrt(res->sumsq) + 1e-6) if max_grad_norm > 0 and
 *          that ratio is below 1, else 1                     (computed in fp64,
 *          then rounded to fp32)
 * and fp32 constants rounded once from fp64: decay = 1 - lr*wd, 1 - beta1,
 * 1 - beta2, bc1 = 1 - beta1^t, bc2 = 1 - beta2^t, each element does, in fp32
 * with one rounding per operation and no fused multiply-add:
 *   g  = (value(grad16[i]) * inv_scale) * coef
 *   p  = master[i] * decay
 *   m  = beta1 * m + (1 - beta1) * g
 *   v  = beta2 * v + (1 - beta2) * (g * g)
 *   p  = p - lr * ((m / bc1) / (sqrt(v / bc2) + eps))
 *   master[i] = p; exp_avg[i] = m; exp_avg_sq[i] = v; param16[i] = round16(p)
 * (round16: nearest, ties to even).
 *   master, exp_avg, exp_avg_sq [count]  device, in/out, fp32
 *   param16[count]                        device, out, 16-bit copy
 *   grad16[count]                         device, in, the reduced gradient
 *   hp                                    host, read during the call
 *   res                                   device, in: written by the check phase
 * Errors: ZERO_EINVAL for NULL pointers, count < 0, hp->step < 1 or an
 * unknown dtype. */
int zero_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                    const void* grad16, int64_t count, int32_t dtype,
                    const zero_adamw_hparams* hp, const zero_step_result* res,
                    hipStream_t stream);

/* ------------------------------------- device-resident step control ---- */
/* The same operations with the per-step scalars read from a device
 * zero_step_control instead of host arguments, so that a whole step can be
 * enqueued (or captured in a graph) once and replayed: the unscale factor is
 * ctl->inv_scale, AdamW's betas and bias corrections are ctl->beta1/2 and
 * ctl->bc1/2 (hp supplies lr, eps, weight_decay and max_grad_norm; hp->step
 * is ignored).  ctl is device memory, read only by these calls. */
int zero_reduce_check_owned_ctl(void* dst, const void* const* srcs, int32_t n_ranks,
                                int64_t count, int32_t dtype, const zero_step_control* ctl,
                                zero_step_result* res, void* workspace, size_t workspace_bytes,
                                int32_t accumulate, hipStream_t stream);

int zero_unscale_check_norm_ctl(const void* grad16, int64_t count, int32_t dtype,
                                const zero_step_control* ctl, zero_step_result* res,
                                void* workspace, size_t workspace_bytes, int32_t accumulate,
                                hipStream_t stream);

int zero_adamw_step_ctl(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                        const void* grad16, int64_t count, int32_t dtype,
                        const zero_adamw_hparams* hp, const zero_step_control* ctl,
                        const zero_step_result* res, hipStream_t stream);

/* Ends a step on the device (one small kernel): with res->overflow set,
 * S = max(S/2, min_scale), clean = 0, skipped += 1; otherwise t += 1,
 * clean += 1 and, when clean reaches window, S = 2S and clean = 0.  Then
 * inv_scale = fp32(1 / (S * D)) and bc1, bc2 for step t + 1 (fp64, rounded
 * once).  Enqueue it after the step's last zero_adamw_step_ctl.
 *   ctl  device, in/out;  res  device, in
 * Errors: ZERO_EINVAL for NULL pointers. */
int zero_step_control_update(zero_step_control* ctl, const zero_step_result* res,
                             hipStream_t stream);

/* --------------------------------------------------------- range lists ---- */
/* One call over several disjoint element ranges of the same buffers: the
 * ranges an owner holds in one step -- its slice of each reduce bucket
 * (ZeRO-2 source walkthrough, section 4.2: gradients reduced bucket by bucket
 * to the partition owners), or, under round-robin ownership (ZeRO optimizer
 * page, "参数分配策略"), every whole tensor it owns.  The result is that of
 * the single-range call on each range in list order (zero_reduce_check_owned
 * with accumulate != 0 after the first, zero_adamw_step per range), except
 * that sumsq adds the per-block partials of all ranges in one fold, so its
 * last bits may differ from the chained calls'.  Ranges that touch (one ends
 * where another begins) are merged, and each merged range is one launch of
 * the single-range kernel; the reduce writes every range's block partials
 * into one workspace and folds the norm once (the chained calls launch a
 * fold and a finalize per range).
 *   ranges[n_ranges]  host array, read during the call; offsets and counts
 *                     >= 0; no element may lie in two ranges (ZERO_EINVAL;
 *                     ZERO_ERANGE when offset + count overflows int64);
 *                     empty ranges are allowed and skipped
 *   ctl               device zero_step_control, or NULL: with ctl the
 *                     unscale factor, betas and bias corrections come from it
 *                     (as in the *_ctl calls) and inv_scale / hp->step are
 *                     ignored
 * Every other argument as in zero_reduce_check_owned / zero_adamw_step; all
 * buffers are indexed by the same element offsets. */

/* Bytes of workspace zero_reduce_check_ranges needs for these ranges (0 for
 * an invalid list). */
size_t zero_range_workspace_bytes(const zero_range* ranges, int32_t n_ranges);

int zero_reduce_check_ranges(void* dst, const void* const* srcs, int32_t n_ranks,
                             const zero_range* ranges, int32_t n_ranges, int32_t dtype,
                             float inv_scale, const zero_step_control* ctl,
                             zero_step_result* res, void* workspace, size_t workspace_bytes,
                             int32_t accumulate, hipStream_t stream);

/* Reduce+check over reduce buckets whose rank contributions arrive in
 * buffers of their own (ZeRO-2 source walkthrough, section 4.2: gradients are
 * reduced bucket by bucket of reduce_bucket_size elements, and each bucket's
 * part of the owner's partition is summed over the N ranks; section 三:
 * reduce_bucket_size 5e8).  Window w is the owner's slice of one bucket: it
 * covers dst[windows[w].offset, windows[w].offset + windows[w].count) and
 * takes rank r's values from srcs[w * n_ranks + r][0 .. count), so each
 * bucket's N slices can sit wherever they arrived (for example back to back
 * in one receive buffer per bucket).  The result is that of
 * zero_reduce_check_owned on each window in list order (accumulate != 0 after
 * the first), except that sumsq adds the per-block partials of all windows in
 * one fold, as in zero_reduce_check_ranges.  Windows are not merged: each
 * non-empty window is one launch of the single-range kernel.
 *   srcs[n_windows * n_ranks]  host array of device pointers; the pointers of
 *                              an empty window are not read
 *   windows[n_windows]         host array, read during the call; disjoint in
 *                              dst, offsets and counts >= 0 (ZERO_EINVAL;
 *                              ZERO_ERANGE when offset + count overflows)
 *   workspace                  at least zero_range_workspace_bytes(windows,
 *                              n_windows) bytes
 * Within a window dst may be the same pointer as one of its rank buffers; no
 * other overlap is allowed.  Every other argument as in
 * zero_reduce_check_ranges. */
int zero_reduce_check_buckets(void* dst, const void* const* srcs, int32_t n_ranks,
                              const zero_range* windows, int32_t n_windows, int32_t dtype,
                              float inv_scale, const zero_step_control* ctl,
                              zero_step_result* res, void* workspace, size_t workspace_bytes,
                              int32_t accumulate, hipStream_t stream);

int zero_adamw_step_ranges(float* master, float* exp_avg, float* exp_avg_sq, void* param16,
                           const void* grad16, const zero_range* ranges, int32_t n_ranges,
                           int32_t dtype, const zero_adamw_hparams* hp,
                           const zero_step_control* ctl, const zero_step_result* res,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */

/*
 * bitopt.h -- C ABI of libbitopt, the MI355X (gfx950) 8-bit block-wise optimizer step.
 *
 * The method: optimizer state is held as one byte per element, a code into a
 * 256-entry non-linear "dynamic exponent" codebook, scaled by one fp32 absmax per
 * block of `blocksize` elements ("8-bit Optimizers via Block-wise Quantization",
 * abstract; the k-bit scaling-laws quote in its citing-papers section).  One step
 * decodes each block, applies the optimizer update in fp32, recomputes the block
 * absmax and re-encodes to the nearest code.  The hyper-parameters mirror the
 * Optimizer2State / Optimizer1State lists of the bitsandbytes "optim_overview"
 * page; the state layout mirrors the state-name table of the "[XPU] Implemented
 * 8bit optimizers in triton #1692" benchmark script; skip_zeros follows "Support
 * skip_zeros in the XPU Triton optimizer kernels #2097".
 *
 * Conventions shared by every entry point
 *   - Every call returns a status code (BITOPT_OK or a negative BITOPT_ERR_*).  On
 *     error, bitopt_last_error() returns a message (per calling thread).  No C++
 *     exception crosses this interface.
 *   - Pointers named as device pointers are caller-owned device memory on the
 *     current HIP device.  The library never allocates, frees or retains caller
 *     memory.  `stream` is a hipStream_t (NULL = the null stream); calls enqueue
 *     work on it and return without waiting (bitopt_multi_plan_build and
 *     bitopt_step_multi, which copy a descriptor table, wait for it).  Launch errors are returned at once;
 *     faults during execution surface at the caller's next synchronisation.
 *   - n == 0 is a successful no-op.  Arguments are checked before anything is
 *     enqueued: n < 0, a NULL pointer that the call needs, an unknown dtype or
 *     optimizer, a blocksize other than 256 or 2048, step < 1, a beta outside
 *     [0, 1), eps < 0, lr < 0 or max_unorm < 0 give BITOPT_ERR_INVALID_ARG.
 *   - Any alignment is accepted; buffers aligned to 16 bytes take the vector path.
 *   - Step calls form their per-step scalars on the host when called and pass them
 *     as kernel arguments: a step captured into a HIP graph replays the step number
 *     (bias corrections, AdEMAMix schedules) it was captured with.  The exception is
 *     bitopt_step_multi_planned_dscalars, whose kernels read them from device memory.
 *   - Calls are stateless and re-entrant.  Fresh state buffers are zero-filled:
 *     codes 0 and absmax 0 decode to zero.
 *   - Element arithmetic is IEEE fp32 (no contraction to FMA, correctly rounded
 *     division and square root); per-step scalars (bias corrections, schedules,
 *     1 - beta, 1 - lr*wd) are formed in double and rounded once to fp32.
 *     Results are deterministic run to run (no atomics).
 */
#ifndef BITOPT_H
#define BITOPT_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define BITOPT_API __attribute__((visibility("default")))
#else
#define BITOPT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BITOPT_OK 0
#define BITOPT_ERR_INVALID_ARG (-1)
#define BITOPT_ERR_UNSUPPORTED (-2)
#define BITOPT_ERR_DEVICE (-3)

/* Element types of parameters, gradients and codec inputs/outputs. */
#define BITOPT_F32 0
#define BITOPT_F16 1
#define BITOPT_BF16 2

/* Optimizers.  ADAM covers Adam and AdamW (decoupled decay when weight_decay > 0).
 * RMSPROP and ADAGRAD are the 1-state optimizers of the 8-bit PR's optimizer table
 * (RMSprop8bit against torch.optim.RMSprop) and of the optimizer overview (Adagrad
 * as its 1-state example), with the torch definitions. */
#define BITOPT_ADAM 0
#define BITOPT_ADEMAMIX 1
#define BITOPT_MOMENTUM 2
#define BITOPT_LION 3
#define BITOPT_RMSPROP 4
#define BITOPT_ADAGRAD 5

/*
 * Hyper-parameters of one step ("optim_overview": Optimizer2State and
 * Optimizer1State argument lists).  Defaults there: lr 1e-3, betas (0.9, 0.999),
 * eps 1e-8, weight_decay 0, max_unorm 0 (off), skip_zeros false, alpha 0,
 * t_alpha / t_beta3 None (here: <= 0).
 *   optimizer     BITOPT_ADAM | BITOPT_ADEMAMIX | BITOPT_MOMENTUM | BITOPT_LION |
 *                 BITOPT_RMSPROP | BITOPT_ADAGRAD
 *   beta1, beta2  Adam/AdEMAMix EMA rates; Momentum uses beta1 as the momentum;
 *                 Lion uses beta1 for the update interpolation, beta2 for its EMA;
 *                 RMSprop uses beta1 as the smoothing constant alpha of square_avg;
 *                 Adagrad uses neither.
 *   beta3, alpha  AdEMAMix slow EMA rate and mixing weight.
 *   t_alpha, t_beta3  AdEMAMix warm-up lengths for alpha and beta3 (<= 0: none).
 *   eps           added to the (bias-corrected, for Adam/AdEMAMix) root of the second
 *                 moment: Adam, AdEMAMix, RMSprop, Adagrad.
 *   weight_decay  decoupled (p *= 1 - lr*wd) for Adam/AdEMAMix/Lion; added to the
 *                 gradient (g + wd*p) for Momentum, RMSprop and Adagrad.
 *   max_unorm     > 0: per block, the update's L2 norm is capped at max_unorm times
 *                 the block's parameter L2 norm.
 *   skip_zeros    != 0: elements whose raw gradient is exactly +-0 keep their
 *                 parameter bits; a block whose every gradient is zero is not
 *                 written at all (codes, absmax, parameters untouched).
 *   blocksize     256 or 2048 elements per absmax block.
 */
typedef struct bitopt_hparams {
    int32_t optimizer;
    float lr, beta1, beta2, beta3, eps, weight_decay, alpha;
    int32_t t_alpha, t_beta3;
    float max_unorm;
    int32_t skip_zeros;
    int32_t blocksize;
} bitopt_hparams;

/* Message describing the last error on the calling thread ("" if none). */
BITOPT_API const char* bitopt_last_error(void);

/* ABI version of this header (increments on incompatible changes). */
BITOPT_API int32_t bitopt_abi_version(void);

/*
 * Host-only.  Writes the 256-entry dynamic-exponent codebook, sorted ascending,
 * into out256 (host memory).  is_signed != 0: the signed map (sign bit, then a run
 * of zero bits selecting the decade 10^-E, an indicator bit and 6-E linear
 * fraction bits; used for first moments).  is_signed == 0: the unsigned map (no
 * sign bit, 7-E fraction bits; used for second moments).  Each pattern stands for
 * the midpoint of its bin; exact 0 and +1.0 are included.  A code is an index
 * into this array.  ("8-bit Optimizers via Block-wise Quantization": abstract and
 * the dynamic-exponent quote among its citing papers.)
 */
BITOPT_API int bitopt_create_dynamic_map(int is_signed, float* out256);

/*
 * Host-only.  The fp32 per-step scalars the step kernels use for `step`, in this
 * order: lr, beta1, beta2, eps, weight_decay, 1-beta1, 1-beta2, 1/(1-beta1^t),
 * 1/sqrt(1-beta2^t), 1-lr*weight_decay, beta3(t), 1-beta3(t), alpha(t), max_unorm.
 * Each is formed in double from the fp32 fields of hp and rounded once.  AdEMAMix
 * ("optim_overview": alpha, t_alpha, t_beta3): alpha(t) = alpha*min(t/t_alpha, 1);
 * beta3(t) moves the slow EMA's half-life linearly from beta1's to beta3's over
 * t_beta3 steps, capped at beta3.  out14: host, 14 floats.
 */
BITOPT_API int bitopt_step_scalars(const bitopt_hparams* hp, int32_t step, float* out14);

/*
 * Block-wise quantization ("8-bit Optimizers via Block-wise Quantization",
 * abstract).  For each block b of `blocksize` elements of x (device, `dtype`):
 * absmax[b] = max |x| over the block's valid elements, then every element gets
 * the index of the nearest qmap entry to x * (1/absmax[b]) (fp32 distance; ties to
 * the lower index; an all-zero block encodes to the code of 0.0).
 *   x        device, n elements of dtype
 *   qmap     device, 256 fp32 sorted ascending
 *   codes    device, n bytes (written)
 *   absmax   device, ceil(n/blocksize) fp32 (written)
 */
BITOPT_API int bitopt_quantize_blockwise(const void* x, int32_t dtype, int64_t n, const float* qmap,
                              int32_t blocksize, uint8_t* codes, float* absmax, void* stream);

/*
 * Block-wise dequantization, as dequantize_blockwise(code, absmax, A, blocksize)
 * in the "#1692" test script: out[i] = qmap[codes[i]] * absmax[i / blocksize],
 * one fp32 multiply, rounded to nearest-even into `dtype`.
 *   codes n bytes, absmax ceil(n/blocksize) fp32, qmap 256 fp32, out n of dtype
 *   (all device).
 */
BITOPT_API int bitopt_dequantize_blockwise(const uint8_t* codes, const float* absmax, const float* qmap,
                                int64_t n, int32_t blocksize, void* out, int32_t dtype, void* stream);

/*
 * Fused 8-bit block-wise step of a 2-state optimizer (Optimizer2State): Adam/AdamW
 * or AdEMAMix.  One pass: decode, update, new absmax, re-encode, write p.
 *   hp      host pointer; optimizer must be BITOPT_ADAM or BITOPT_ADEMAMIX
 *   step    1-based step count t (bias corrections and schedules use it)
 *   p       device, n elements of dtype (read and written)
 *   g       device, n elements of dtype (read)
 *   state1  device uint8 codes of the first moment: n bytes (Adam: exp_avg);
 *           AdEMAMix: 2n bytes, fast EMA m1 then slow EMA m2
 *   state2  device uint8 codes of the second moment, n bytes (exp_avg_sq / nu)
 *   absmax1 device fp32, nb = ceil(n/blocksize) entries (AdEMAMix: 2*nb, m1's then m2's)
 *   absmax2 device fp32, nb entries
 *   qmap1   device fp32[256], signed map (shared by m1 and m2)
 *   qmap2   device fp32[256], unsigned map
 */
BITOPT_API int bitopt_step_8bit_blockwise_2state(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                      int32_t dtype, int64_t n, uint8_t* state1, uint8_t* state2,
                                      float* absmax1, float* absmax2, const float* qmap1,
                                      const float* qmap2, void* stream);

/*
 * Fused 8-bit block-wise step of a 1-state optimizer (Optimizer1State): Momentum
 * (state1 = momentum_buffer), Lion (state1 = exp_avg), RMSprop (state1 =
 * square_avg) or Adagrad (state1 = sum of squared gradients).  Arguments as above
 * with one state: state1 n bytes, absmax1 nb fp32, qmap1 the map of the state --
 * the signed map for Momentum and Lion; RMSprop's and Adagrad's state is never
 * negative, and the unsigned map spends all 256 codes on it.
 */
BITOPT_API int bitopt_step_8bit_blockwise_1state(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                      int32_t dtype, int64_t n, uint8_t* state1, float* absmax1,
                                      const float* qmap1, void* stream);

/*
 * 32-bit steps: the same updates with fp32 states and no codec -- the path for
 * tensors below min_8bit_size ("optim_overview": min_8bit_size, default 4096) and
 * the 32-bit optimizers the 8-bit ones are compared against.
 *   2-state: state1 fp32 n (Adam: m; AdEMAMix: 2n, m1 then m2), state2 fp32 n (v / nu)
 *   1-state: state1 fp32 n
 * skip_zeros leaves the states of zero-gradient elements untouched; max_unorm
 * groups elements in blocks of hp->blocksize.
 */
BITOPT_API int bitopt_step_32bit_2state(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                             int32_t dtype, int64_t n, float* state1, float* state2, void* stream);
BITOPT_API int bitopt_step_32bit_1state(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                             int32_t dtype, int64_t n, float* state1, void* stream);

/*
 * One tensor of a multi-tensor step (host-side descriptor; every pointer inside is
 * caller-owned device memory):
 *   p, g      n elements of dtype
 *   state1    is_8bit: uint8 codes, n bytes (AdEMAMix 2n); else fp32 states, n (AdEMAMix 2n)
 *   state2    2-state optimizers: uint8 codes / fp32 states, n; 1-state: NULL
 *   absmax1   is_8bit: ceil(n/blocksize) fp32 (AdEMAMix 2x); else NULL
 *   absmax2   is_8bit and 2-state: ceil(n/blocksize) fp32; else NULL
 *   is_8bit   0 selects the 32-bit step, as for tensors below min_8bit_size
 *             ("optim_overview": min_8bit_size, default 4096)
 */
typedef struct bitopt_tensor {
    void* p;
    const void* g;
    void* state1;
    void* state2;
    float* absmax1;
    float* absmax2;
    int64_t n;
    int32_t dtype;
    int32_t is_8bit;
} bitopt_tensor;

/*
 * Non-block-wise ("tensor-wide") 8-bit step: each state keeps ONE absmax for the
 * whole tensor instead of one per block -- the form that block-wise quantization
 * ("8-bit Optimizers via Block-wise Quantization", abstract) improves on, kept here
 * to measure that claim.  The same update, codes and maps as the block-wise steps:
 *   absmax1  device fp32, 1 entry (AdEMAMix: 2, m1's then m2's)
 *   state2, absmax2 (1 entry), qmap2  2-state optimizers; NULL for 1-state ones
 *   hp->blocksize must be 0 (one block spanning the tensor); hp->max_unorm > 0 caps
 *            the norm of the whole tensor's update at max_unorm times the norm of
 *            its parameters (one block of n elements)
 *   workspace device memory of at least bitopt_tensorwise_workspace_bytes() bytes,
 *            4-byte aligned, caller-owned and overwritten; calls that may run
 *            concurrently must not share one
 * The new absmax depends on every element, so the step is three launches on
 * `stream`: a pass that reads g, the codes and (Momentum, RMSprop, Adagrad, or
 * with max_unorm) p and leaves each group's max |new state| (and sums of squares of
 * update and parameters) in the workspace; a one-group reduction of those; a pass
 * that reads everything again, writes p, encodes with the tensor-wide scale and
 * writes codes and absmax.  The results equal the block-wise step with one block
 * of n elements (deterministic: no atomics).
 */
BITOPT_API int64_t bitopt_tensorwise_workspace_bytes(void);
BITOPT_API int bitopt_step_8bit_tensorwise(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                           int32_t dtype, int64_t n, uint8_t* state1, uint8_t* state2,
                                           float* absmax1, float* absmax2, const float* qmap1,
                                           const float* qmap2, void* workspace, void* stream);

/*
 * The tensor-wide step without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments and results are those of bitopt_step_8bit_tensorwise;
 * its partial results go to the library's own scratch array instead: a file-scope
 * device array of bitopt_tensorwise_scratch_bytes() bytes (32.8 KB) on each GPU the
 * library runs on, held until the process ends.  The step needs that much for any n
 * (pass 1 has at most 1024 groups), so no size exceeds it.  The call allocates nothing
 * (no hipMalloc, no library allocation); its first call on a device looks the array's
 * address up.  Every call on one GPU shares that GPU's array: calls that may overlap
 * on one GPU (other streams, other threads) race and must be ordered by the caller.
 * Nothing in the array needs to start at zero (each pass writes what it reads).
 */
BITOPT_API int bitopt_step_8bit_tensorwise_noalloc(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                                   int32_t dtype, int64_t n, uint8_t* state1, uint8_t* state2,
                                                   float* absmax1, float* absmax2, const float* qmap1,
                                                   const float* qmap2, void* stream);
BITOPT_API int64_t bitopt_tensorwise_scratch_bytes(void);

/*
 * Optimizer state outside HBM ("paged" state: the optimizer overview's is_paged, the
 * Paged*8bit optimizers of the 8-bit PR's optimizer table).  Pinned host memory,
 * mapped into the GPU's address space with the same address, so the state arrays of
 * any step (codes, absmax, fp32 states) may live there: the kernels read and write it
 * over the host link instead of HBM, unchanged.  Paging state in or out is a copy
 * between such a buffer and device memory (e.g. hipMemcpyAsync) between steps.
 *   bytes  > 0; *ptr receives the address (usable by the host and in every step call)
 *   Returns BITOPT_ERR_DEVICE if the allocation fails, BITOPT_ERR_UNSUPPORTED if the
 *   runtime maps it at a different device address.  The memory is caller-owned until
 *   passed to bitopt_host_state_free (after the last step using it has completed).
 */
BITOPT_API int bitopt_host_state_alloc(int64_t bytes, void** ptr);
BITOPT_API int bitopt_host_state_free(void* ptr);

/*
 * Paged state, staged: one 8-bit block-wise step (2-state or 1-state) whose codes and
 * absmax live in host memory (bitopt_host_state_alloc or other pinned memory; the
 * optimizer overview's is_paged, the Paged*8bit optimizers of the 8-bit PR).  The
 * tensor is cut into chunks of whole blocks; for each chunk the state is paged into
 * one of two HBM staging buffers on `h2d_stream`, stepped on `stream` by the same
 * kernels as bitopt_step_8bit_blockwise_*, and paged back out on `d2h_stream`, so
 * the copy-in of the next chunk and the write-back of the previous one overlap the
 * step of the current one (event ordering, no host waits; the call enqueues and
 * returns).  Results are bit-identical to the device-resident step.
 *   host_state1/2, host_absmax1/2  host memory laid out as the device-resident call's
 *            state1/2, absmax1/2 (state2, absmax2, qmap2: NULL for 1-state optimizers)
 *   p, g     device, n elements of dtype
 *   staging  device, 256-byte aligned, staging_bytes long; chunk size = the largest
 *            multiple of 4096 elements whose two buffers fit (at least
 *            bitopt_paged_staging_bytes(hp, 4096) bytes); overwritten
 *   h2d_stream, d2h_stream, stream  three distinct streams.  Work already on
 *            `stream` completes before the host state is read; `stream` completes
 *            only after every write-back.  Calls that share staging or copy streams
 *            must be ordered on `stream`.
 * Errors: as the per-tensor calls; a staging buffer below the minimum, misaligned, or
 * streams that are not distinct give INVALID_ARG.
 */
BITOPT_API int64_t bitopt_paged_staging_bytes(const bitopt_hparams* hp, int64_t chunk_elems);
BITOPT_API int bitopt_step_8bit_paged(const bitopt_hparams* hp, int32_t step, void* p, const void* g,
                                      int32_t dtype, int64_t n, uint8_t* host_state1, uint8_t* host_state2,
                                      float* host_absmax1, float* host_absmax2, const float* qmap1,
                                      const float* qmap2, void* staging, int64_t staging_bytes,
                                      void* h2d_stream, void* d2h_stream, void* stream);

/*
 * Paged state, cached: an HBM page pool in front of host-resident 8-bit state (the
 * optimizer overview's is_paged and the 8-bit PR's Paged*8bit optimizers keep state in
 * memory that lives on the GPU while it fits and moves to host memory under pressure;
 * here the library does that paging explicitly).  A page is the state of one range of
 * page_elems elements of one tensor (its codes and absmax, the layout of a staging
 * chunk); a frame is HBM room for one page.  A pooled step looks every page of its
 * tensor up (key: host_state1 and the page index): a resident page is stepped where it
 * lies; a missing one takes a free frame or the least recently used one (whose page is
 * first written back to its host buffers if stepped since), is copied in, then stepped.
 * When every page fits, steps after the first copy nothing and run at the speed of the
 * device-resident step; when they do not, each step pages its state through the frames.
 * Results are bit-identical to the device-resident step.  The host buffers are current
 * only after bitopt_page_pool_flush (and its stream's completion).
 *
 * Copies run on two streams the pool owns (default priority), ordered by events
 * against the step streams; no call waits on the host.  A pool is not thread-safe: one
 * host thread at a time.  It belongs to the device current at its creation.
 */
typedef struct bitopt_page_pool bitopt_page_pool;

/* Bytes of one frame for pages of page_elems elements (a positive multiple of 4096), or
 * < 0 for invalid arguments. */
BITOPT_API int64_t bitopt_page_pool_frame_bytes(const bitopt_hparams* hp, int64_t page_elems);

/*
 *   hp           optimizer and blocksize of every tensor the pool will hold (fixes the
 *                page layout); the other fields are not used
 *   page_elems   a positive multiple of 4096
 *   frames       device, 256-byte aligned, frames_bytes long, caller-owned; holds
 *                floor(frames_bytes / frame_bytes) frames, at least 2 (at most 2^20).
 *                In use by the pool until bitopt_page_pool_destroy returns
 *   *pool        receives the pool (a host object)
 * Errors: INVALID_ARG for the above; DEVICE if its streams or events cannot be made.
 */
BITOPT_API int bitopt_page_pool_create(const bitopt_hparams* hp, int64_t page_elems, void* frames,
                                       int64_t frames_bytes, bitopt_page_pool** pool);
/* Waits for the pool's copies, then releases its streams, events and host object.
 * Writes nothing back: flush first to keep the state.  NULL is accepted. */
BITOPT_API int bitopt_page_pool_destroy(bitopt_page_pool* pool);

/*
 * One 8-bit block-wise step (2-state or 1-state, as bitopt_step_8bit_blockwise_*) on a
 * tensor whose state lives in host buffers (bitopt_host_state_alloc or other pinned
 * memory, laid out as the device-resident call's state1/2, absmax1/2; state2, absmax2,
 * qmap2 NULL for 1-state optimizers), through `pool`.  p, g, qmap1/2: device.  Work
 * already on `stream` (e.g. the gradient) precedes the step; calls enqueue and return.
 * A host_state1 already in the pool must come with the same companion buffers and n.
 * Host buffers of different tensors must not overlap.  Before host buffers are freed
 * or reused for another tensor, flush with evict = 1.
 * Errors: as the per-tensor calls; INVALID_ARG when hp's optimizer or blocksize differs
 * from the pool's, for another current device, or for mismatched companion buffers.
 * After a DEVICE error the pool's bookkeeping is undefined: destroy it.
 */
BITOPT_API int bitopt_step_8bit_pooled(bitopt_page_pool* pool, const bitopt_hparams* hp, int32_t step, void* p,
                                       const void* g, int32_t dtype, int64_t n, uint8_t* host_state1,
                                       uint8_t* host_state2, float* host_absmax1, float* host_absmax2,
                                       const float* qmap1, const float* qmap2, void* stream);

/*
 * Writes every page stepped since its last write-back to its host buffers; `stream`
 * completes only after all of them (work already on `stream` precedes them).  evict
 * != 0 also empties the pool (the next step on any tensor copies its state in again).
 */
BITOPT_API int bitopt_page_pool_flush(bitopt_page_pool* pool, int32_t evict, void* stream);

/* out4 = {resident pages, page-ins, write-backs, resident hits} since creation. */
BITOPT_API int bitopt_page_pool_stats(const bitopt_page_pool* pool, int64_t* out4);

/* Bytes of device workspace a multi-tensor step needs for `count` tensors (< 0 if count < 0). */
BITOPT_API int64_t bitopt_multi_workspace_bytes(int32_t count);

/*
 * Multi-tensor steps: one optimizer step over many tensors ("optim_overview": one
 * optimizer holds every parameter of a model; tensors below min_8bit_size keep
 * 32-bit states).  Each tensor gets the same result, bit for bit, as the per-tensor
 * 8-bit or 32-bit entry point (by is_8bit) with the same hp and step.  Tensors are
 * grouped by (dtype, is_8bit); each group is one kernel launch over all of its
 * tiles, so hundreds of small tensors cost a few launches.
 *
 * A plan holds the grouping on the host and the tensors' device descriptors (80 B
 * per tensor) in a caller-owned device workspace.  It is built once per set of
 * tensors (bitopt_multi_plan_build: validates every tensor, writes the workspace,
 * waits for `stream`) and then stepped any number of times
 * (bitopt_step_multi_planned: kernel launches only -- it enqueues and returns, and
 * may be captured into a HIP graph).  The plan stays valid while the workspace and
 * every tensor buffer it names stay allocated at the same addresses.
 */
#define BITOPT_MULTI_MAX_LAUNCHES 64
typedef struct bitopt_multi_launch {
    int32_t kind8;      /* 1: 8-bit states, 0: 32-bit states */
    int32_t dtype;      /* parameter dtype of the group */
    int32_t first;      /* first descriptor of the launch in the workspace table */
    int32_t count;      /* descriptors in the launch */
    int64_t tiles;      /* wave tiles over the launch's tensors */
} bitopt_multi_launch;

typedef struct bitopt_multi_plan {
    int32_t optimizer;  /* hp->optimizer and hp->blocksize the plan was built for */
    int32_t blocksize;
    int32_t count;      /* descriptors written (tensors with n > 0) */
    int32_t nlaunch;
    void* workspace;    /* device descriptor table */
    bitopt_multi_launch launch[BITOPT_MULTI_MAX_LAUNCHES];
} bitopt_multi_plan;

/*
 * Build a plan (host struct `plan`, caller-owned) for `count` tensors (host array;
 * n == 0 entries are skipped) and write their device descriptors into `workspace`
 * (device, at least bitopt_multi_workspace_bytes(count) bytes, 16-byte aligned).
 * Only hp->optimizer and hp->blocksize shape the plan.  The descriptor copy is
 * enqueued on `stream` and waited for before the call returns, so `tensors` may be
 * reused at once.  Errors: as the per-tensor calls, checked for every tensor before
 * anything is enqueued; a small or misaligned workspace gives INVALID_ARG; more than
 * BITOPT_MULTI_MAX_LAUNCHES launches (beyond ~58000 tensors) gives UNSUPPORTED.
 */
BITOPT_API int bitopt_multi_plan_build(const bitopt_hparams* hp, const bitopt_tensor* tensors, int32_t count,
                                       void* workspace, int64_t workspace_bytes, bitopt_multi_plan* plan,
                                       void* stream);

/*
 * One step over the tensors of a plan: one kernel launch per group on `stream`,
 * nothing else (no copies, no waits).  hp must have the plan's optimizer and
 * blocksize; the other fields (and step) may change from call to call.
 *   qmap1/2  device codebooks as for the per-tensor calls (needed when any tensor is
 *            8-bit; qmap2 for 2-state optimizers)
 * Graph capture: the per-step scalars (bias corrections, schedules) are formed on
 * the host from hp and step when the call is made and passed as kernel arguments,
 * so a captured call replays the step number and hyper-parameters it was captured
 * with; capture one graph per step value, call eagerly, or use the device-scalar form
 * below.  (The same holds for every other step entry point.)
 */
BITOPT_API int bitopt_step_multi_planned(const bitopt_multi_plan* plan, const bitopt_hparams* hp, int32_t step,
                                         const float* qmap1, const float* qmap2, void* stream);

/*
 * The per-step scalars in device form: bitopt_device_scalars_bytes() bytes (at most
 * 64) that bitopt_device_scalars_write fills, on the host, for (hp, step) -- the bias
 * corrections of the optimizer pages' update rules and the AdEMAMix schedules, as the
 * other entry points form them.  out: host memory of out_bytes bytes.
 */
BITOPT_API int64_t bitopt_device_scalars_bytes(void);
BITOPT_API int bitopt_device_scalars_write(const bitopt_hparams* hp, int32_t step, void* out, int64_t out_bytes);

/*
 * A planned step whose kernels read the per-step scalars from device memory:
 * `scalars` (device, 16-byte aligned, bitopt_device_scalars_bytes() bytes, written by
 * the caller from bitopt_device_scalars_write with this hp, e.g. by a copy on `stream`)
 * is read when the kernels run, so a graph that captures this call steps with whatever
 * the buffer holds at each replay: update it before each replay (a training loop: write
 * step t's scalars, copy them in, replay).  hp selects the kernels (optimizer, blocksize,
 * skip_zeros, whether max_unorm > 0) and must equal the hp the scalars were written
 * with in those fields.  The results equal bitopt_step_multi_planned's for that step.
 * Errors: as bitopt_step_multi_planned; NULL or misaligned scalars give INVALID_ARG.
 */
BITOPT_API int bitopt_step_multi_planned_dscalars(const bitopt_multi_plan* plan, const bitopt_hparams* hp,
                                                  const void* scalars, const float* qmap1, const float* qmap2,
                                                  void* stream);

/*
 * Plan and step in one call: bitopt_multi_plan_build followed by
 * bitopt_step_multi_planned.  It waits for the stream once (the descriptor copy), so a
 * training loop builds a plan once and calls bitopt_step_multi_planned per step.
 */
BITOPT_API int bitopt_step_multi(const bitopt_hparams* hp, int32_t step, const bitopt_tensor* tensors,
                                 int32_t count, const float* qmap1, const float* qmap2, void* workspace,
                                 int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITOPT_H */

/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA frozen-NF4 linear layer.
 *
 * The layer is the two-term forward of "QLoRA는 어떻게 65B 모델을 GPU 한 장에
 * 올렸나" (section "QLoRA의 수식"):
 *
 *     h = dequant(W_NF4, c_block) x + (alpha/r) B A x
 *
 * with tokens as rows: x [T, d_in], W [d_out, d_in], A [r, d_in], B [d_out, r],
 * h [T, d_out]. The base weight is stored as 4-bit NF4 indices in blocks of 64
 * with a per-block absmax scale that is itself re-quantized to 8 bits against a
 * per-group float32 maximum ("48GB GPU Fine-Tuning a 65B Model", section
 * "Quantization Keeps the Patterns and Reduces Bits per Number"; the
 * double-quantization paragraph and reconstruction equation of the first page,
 * section "메모리 회계"). Compute is bf16 with float32 accumulation.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP), row-major, 16-byte aligned,
 *     except where a comment says "host".
 *   - The library allocates no memory. The caller owns every buffer; inputs must
 *     stay alive and unmodified until the stream work has completed.
 *   - Work is enqueued asynchronously on `stream` (0 = the legacy default stream).
 *   - Arguments are validated on the host before anything is enqueued. On any
 *     error the call returns a negative status and writes no output byte.
 *   - Shapes: d_in % 64 == 0, d_out % 16 == 0, both <= QLORA_MAX_DIM, and
 *     fewer than 2^32 blocks (d_out * d_in < 2^38);
 *     1 <= T <= QLORA_MAX_TOKENS; 0 <= r <= 256 with r % 8 == 0.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Calls that run concurrently (other streams or threads) must not share a
 *     workspace; with distinct workspaces they may overlap freely. No kernel
 *     depends on another launch finishing, or on all of its own workgroups
 *     being resident at once: where workgroups of one launch wait for each
 *     other, a wait that runs out of time (about 200 us) takes a path that
 *     needs no one else and gives the same bits (see qlora_workspace_fallbacks).
 *   - The header is plain C: it needs only hip_runtime_api.h for hipStream_t.
 *     A host compiler other than hipcc defines __HIP_PLATFORM_AMD__ for that
 *     header, as `hipconfig --cpp_config` prints.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_BLOCK 64   /* weights per absmax block                          */
#define QLORA_GROUP 256  /* blocks per double-quant group (one float32 S_g)    */
#define QLORA_MAX_RANK 256
#define QLORA_MAX_DIM (1 << 20)          /* d_in, d_out upper bound            */
#define QLORA_MAX_TOKENS (1 << 24)       /* T upper bound                      */
#define QLORA_WS_COUNTER_BYTES 65536     /* zeroed counter region of a workspace */
#define QLORA_STATIC_SCRATCH_BYTES (1u << 20) /* scratch of qlora_forward_noalloc per GPU */

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,      /* a required pointer is NULL                     */
  QLORA_ERR_SHAPE = -2,     /* d_in % 64 != 0, a size < 1, or r out of range  */
  QLORA_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned               */
  QLORA_ERR_WORKSPACE = -4, /* ws_bytes < qlora_workspace_bytes(...)          */
  QLORA_ERR_DTYPE = -5,     /* unknown dtype enum                             */
  QLORA_ERR_HIP = -6,       /* a kernel launch failed                         */
  QLORA_ERR_INTERNAL = -7,  /* the levels compiled into the kernels differ from
                               the table derived at load (never expected)      */
  QLORA_ERR_MEMORY = -8,    /* a pointer is neither device memory nor pinned
                               (hipHostMalloc) host memory                     */
  QLORA_ERR_VALUE = -9,     /* a hyperparameter is out of range                */
  QLORA_ERR_SCRATCH = -10   /* qlora_forward_noalloc: T > 16, or more scratch
                               than QLORA_STATIC_SCRATCH_BYTES                 */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

/*
 * A quantized frozen weight W [d_out, d_in] (d_in % 64 == 0), n = d_out*d_in,
 * nblocks = n/64, ngroups = ceil(nblocks/256). Blocks are 64 consecutive
 * weights of the row-major flattening (so a block never straddles a row);
 * groups are 256 consecutive blocks (they may straddle rows).
 *   codes  [n/2]      u8   4-bit codebook indices; each run of 8 consecutive
 *                          weights e0..e7 is one little-endian 32-bit word whose
 *                          byte i holds e_i (low nibble) and e_(i+4) (high nibble)
 *   qscale [nblocks]  u8   8-bit code q2 of each block scale, 0..255
 *   smax   [ngroups]  f32  per-group maximum S_g of the block scales
 * Restored weight: w_hat = bf16( c[q] * (q2/256 * S_g) ), each product rounded
 * to float32 first (reconstruction equation of the "메모리 회계" section).
 *
 * Absmax-only storage (4.5 bits per weight: the same page and section, NF4
 * paragraph, before double quantization) is selected by qscale == NULL:
 *   smax   [nblocks]  f32  the block absmax s_k itself
 * and w_hat = bf16( c[q] * s_k ). The codes are the same as with double
 * quantization. Every entry point that takes a weight accepts either storage;
 * absmax-only storage needs nblocks * 4 < 2^31 bytes of scales (else SHAPE).
 */
typedef struct {
  int64_t d_out;
  int64_t d_in;
  uint8_t *codes;
  uint8_t *qscale;
  float *smax;
} qlora_nf4_weight;

/*
 * Quantize W once (a load-time step in the pages' training snippet, "무엇을
 * 돌렸나" of the GPU-fit page).
 *   W        device, [d_out, d_in], float32 or bf16 (w_dtype)
 *   out      host struct naming the three output buffers (sizes above)
 *   flags    device u32, nullable; bit 0 is OR-ed in when a non-finite weight is
 *            seen (the codes are then unspecified)
 * Per block: s = max|w|; each w/s (IEEE float32 divide) takes the index of the
 * nearest NF4 level, ties to the lower index; s = 0 gives index 7 (exact zero).
 * Per group: S = max s; q2 = min(255, rint(fl32(s/S)*256)); S = 0 gives q2 = 0.
 * With out->qscale == NULL (absmax-only storage) s itself goes to smax[block]
 * and there is no group step. Bit-exact with the CPU oracle.
 */
int qlora_quantize(const void *W, int w_dtype, const qlora_nf4_weight *out, uint32_t *flags,
                   hipStream_t stream);

/*
 * Quantize several weights at once, as a model load does for every projection:
 * the results are those of `count` qlora_quantize calls (bit for bit), but up
 * to 32 weights share one launch, so small weights do not each pay a launch
 * and a partly idle tail.
 *   W      host array of `count` device pointers, all of dtype w_dtype
 *   out    host array of `count` structs naming each weight's output buffers
 *          (double-quant and absmax-only storage may be mixed)
 *   flags  as for qlora_quantize, shared by all weights
 * Every job's arguments are checked before anything is launched (an argument
 * error writes nothing). Errors: as qlora_quantize, and SHAPE for count < 0.
 */
int qlora_quantize_many(const void *const *W, int w_dtype, const qlora_nf4_weight *out, int32_t count,
                        uint32_t *flags, hipStream_t stream);

/*
 * Restore the full weight (for checking, merging or export).
 *   out  device, [d_out, d_in], float32 (the unrounded float32 product) or bf16.
 */
int qlora_dequantize(const qlora_nf4_weight *W, int out_dtype, void *out, hipStream_t stream);

/*
 * Merge a trained adapter into the restored weight, for export ("48GB GPU
 * Fine-Tuning a 65B Model: Where QLoRA Saves GPU Memory", section "QLoRA Puts
 * the Two Methods in Different Places": A and B cannot be added to the 4-bit
 * weights and are merged into the restored 16-bit weights).
 *   A    device bf16 [r, d_in], B device bf16 [d_out, r]; r = 0 or A = B = NULL
 *        gives the plain bf16 restore
 *   out  device bf16 [d_out, d_in], written in full; 16-byte aligned
 * out = bf16( fl32(w_hat + s * (B A)) ) with s = alpha / r in float32, B A
 * accumulated in float32, s (B A) + w_hat formed by one fused multiply-add and
 * one round-to-nearest-even to bf16 at the end: within one bf16 unit in the
 * last place of the exactly rounded merge, plus the float32 error of forming
 * the sum (2^-24 (|w_hat| + (r+2) s sum_j |B_j||A_j|), which matters only
 * where w_hat and s B A nearly cancel). The weight buffers are
 * only read. Errors: NULL, SHAPE (r outside 0..256 or r % 8 != 0), ALIGN,
 * HIP (launch failure); nothing is written on a validation error.
 */
int qlora_merge(const qlora_nf4_weight *W, const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                uint16_t *out, hipStream_t stream);

/*
 * Forward h = x W_hat^T + (alpha/r) (x A^T) B^T ("QLoRA의 수식").
 *   x      device bf16 [T, d_in]
 *   A, B   device bf16 [r, d_in], [d_out, r]; both NULL, or r == 0, means base only
 *   h      device bf16 [T, d_out] (overwritten)
 *   u_out  device f32 [T, r], nullable: receives u = x A^T for the backward
 *   ws     device workspace of at least qlora_workspace_bytes(d_out, d_in, T, r)
 *          bytes. Its first QLORA_WS_COUNTER_BYTES bytes are u32 counters that
 *          must be zero before the first use of the workspace; every call leaves
 *          them zero again, except the last one, which counts the waits that ran
 *          out of time (qlora_workspace_fallbacks; the output never depends on
 *          it). The rest of the workspace needs no initialisation.
 * T <= 16 runs one weight-streaming kernel (the adapter intermediate is formed
 * by the last workgroups of the same launch); larger T runs the MFMA GEMM.
 */
int qlora_forward(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A,
                  const uint16_t *B, int32_t r, float alpha, uint16_t *h, float *u_out, void *ws,
                  size_t ws_bytes, hipStream_t stream);

/*
 * Several independent forwards of T <= 16 tokens each (the weight-streaming
 * regime) in as few launches as possible: per job, the qlora_forward of
 * "QLoRA의 수식" with that job's weight, input, adapter and outputs. Jobs that
 * share a kernel variant (x of at most 136 KB or not; d_in/64 a multiple of 4 or
 * not) run in one launch, up to 8 of them, and pay its start and its tail once;
 * the compute units are shared out by weight bytes. For projections that
 * cannot be stacked into one weight: separate q, k, v or gate, up weights with
 * their own adapters, or the same step's calls of several models or adapters.
 *   jobs   host array of `count` (1 <= count <= QLORA_MAX_FORWARD_JOBS) job
 *          structs; each job's fields are qlora_forward's arguments, with T <= 16
 *   ws     device workspace of at least qlora_forward_many_workspace_bytes(count)
 *          bytes, its counter region zero as for qlora_forward
 * The jobs must be independent: no job's output may overlap another job's input
 * or output. u_out is bit-identical to qlora_forward's; h differs from it at
 * most in the float32 summation order of the K segments (a job's share of the
 * compute units decides which wave sums which segments), and is the same bits
 * on every call with the same jobs. Every job is checked before anything is
 * launched (an argument error writes nothing). Errors: those of qlora_forward;
 * SHAPE for a job with T > 16 or a count outside 1..QLORA_MAX_FORWARD_JOBS.
 */
typedef struct {
  const qlora_nf4_weight *W;
  const uint16_t *x;   /* device bf16 [T, d_in] */
  int64_t T;           /* 1..16 */
  const uint16_t *A;   /* device bf16 [r, d_in] or NULL */
  const uint16_t *B;   /* device bf16 [d_out, r] or NULL */
  int32_t r;
  float alpha;
  uint16_t *h;         /* device bf16 [T, d_out], overwritten */
  float *u_out;        /* device f32 [T, r] or NULL */
} qlora_forward_job;
#define QLORA_MAX_FORWARD_JOBS 64
int qlora_forward_many(const qlora_forward_job *jobs, int32_t count, void *ws, size_t ws_bytes,
                       hipStream_t stream);
/* Workspace bytes of qlora_forward_many for `count` jobs (0 for a count outside 1..QLORA_MAX_FORWARD_JOBS). */
size_t qlora_forward_many_workspace_bytes(int32_t count);

/*
 * Backward through the frozen restored weight ("QLoRA의 수식", "명제 1"):
 *   v  = dY B
 *   dX = dY W_hat + (alpha/r) v A        device bf16 [T, d_in], nullable
 *   dA = (alpha/r) v^T x                 device f32 [r, d_in], nullable, overwritten
 *   dB = (alpha/r) dY^T u,  u = x A^T    device f32 [d_out, r], nullable, overwritten
 *   u_saved  device f32 [T, r] from qlora_forward's u_out, nullable (then recomputed)
 *   x        needed only for dA, and for dB when u_saved is NULL: with a frozen A
 *            (LoRA-FA, "8GB, 12GB, 16GB, 24GB GPU에서 몇 B 모델까지 LoRA 학습이
 *            될까", section "LoRA 변형을 바꿔도 답이 같은 이유": the layer input
 *            is not kept) pass x = NULL, dA = NULL and u_saved.
 * The codes/qscale/smax buffers are only read: no gradient flows into W.
 * With r == 0 only dX is produced (dA, dB must be NULL).
 */
int qlora_backward(const qlora_nf4_weight *W, const uint16_t *x, const uint16_t *dY, int64_t T,
                   const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                   const float *u_saved, uint16_t *dX, float *dA, float *dB, void *ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * One AdamW step for adapter parameters whose optimizer state is paged out to
 * host memory (first page, the paged-optimizer entry of section "메모리 회계":
 * the adapters' Adam state m, v goes to CPU pinned memory and the update runs
 * beside the backward on another stream). Per element, in float32, with
 * decoupled weight decay (Loshchilov and Hutter's AdamW):
 *     p <- p (1 - lr wd);  m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
 *     p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 *   hp      host struct: lr >= 0, 0 <= beta1, beta2 < 1, eps > 0, weight_decay >= 0
 *   step    t >= 1 (the bias corrections are formed in float64, passed as float32)
 *   n       number of elements (>= 0; 0 does nothing)
 *   grad    device f32 [n] (e.g. qlora_backward's dA or dB)
 *   master  f32 [n] float32 copy of the parameters, updated in place
 *   m, v    f32 [n] first and second moments, updated in place
 *   param   device bf16 [n], nullable: receives bf16(master) for the layer
 * master, m and v may be device memory or pinned host memory (hipHostMalloc,
 * e.g. torch pin_memory=True); the kernel reads and writes host memory in
 * place. Every pointer 16-byte aligned. Errors: NULL, VALUE (hyperparameters,
 * step < 1), SHAPE (n < 0), ALIGN, MEMORY (pageable host memory), HIP.
 */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
} qlora_adamw_hparams;

int qlora_adamw_step(const qlora_adamw_hparams *hp, int64_t step, int64_t n, const float *grad, float *master,
                     float *m, float *v, uint16_t *param, hipStream_t stream);

/*
 * The same AdamW step run by the host CPU, the page's own placement of the
 * paged optimizer's update ("메모리 회계": the CPU runs the optimizer step on
 * the state in pinned CPU memory while the GPU goes on with the backward). The
 * caller copies grad to host memory first and param back to the device after:
 * plain DMA copies, so the GPU's compute units never run the update.
 *   grad    host f32 [n];  master, m, v  host f32 [n], updated in place
 *   param   host bf16 [n], nullable: receives bf16(master) (round to nearest even)
 *   threads worker threads to use (<= 0: all of the pool, at most 16)
 * The per-element arithmetic is qlora_adamw_step's, in float32 (results agree
 * to rounding). Blocks until done; calls from several host threads take turns.
 * Errors: NULL, VALUE (hyperparameters, step < 1), SHAPE (n < 0).
 */
int qlora_adamw_step_host(const qlora_adamw_hparams *hp, int64_t step, int64_t n, const float *grad, float *master,
                          float *m, float *v, uint16_t *param, int32_t threads);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qlora_forward without a
 * workspace argument, for the weight-streaming regime of T <= 16 tokens (the
 * decode-shaped calls of a serving loop). Its scratch -- the counter region and
 * the tagged exchange of the adapter intermediate, about 200 KB at r = 256 --
 * is one static device array of QLORA_STATIC_SCRATCH_BYTES per GPU, held until
 * the process ends; the library takes its address once per device
 * (hipGetSymbolAddress) on the first call there and clears it with a fill
 * kernel on `stream`. Arguments, layouts and results are those of
 * qlora_forward, bit for bit. The call allocates nothing. Calls that overlap
 * on one GPU (other streams, other threads) share that array and race:
 * serialize them. Errors: those of qlora_forward; SCRATCH for T > 16 or a call
 * the array cannot hold; HIP when the array's address cannot be had. Nothing
 * is enqueued on an error.
 */
int qlora_forward_noalloc(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A,
                          const uint16_t *B, int32_t r, float alpha, uint16_t *h, float *u_out,
                          hipStream_t stream);

/*
 * Host: the number of waits that ran out of time on this workspace since it
 * was zeroed (the last u32 of its counter region). Such a wait means another
 * launch held the compute units the awaited workgroups needed; the results are
 * the same, only slower. Copies one word on `stream` and synchronizes it.
 * Errors: NULL, HIP.
 */
int qlora_workspace_fallbacks(const void *ws, uint32_t *count, hipStream_t stream);

/*
 * Host, a testing aid: the bounded waits of later calls on this workspace give
 * up after `ticks` ticks of the 100 MHz constant clock instead of the built-in
 * 20000 (about 200 us); 0 restores the built-in limit. The limit is the u32
 * just before the fallback count. With ticks = 1 every wait that does not
 * succeed at once takes its fallback path (see qlora_workspace_fallbacks),
 * so a test can check that those paths give the same bits. Sets one word on
 * `stream` and synchronizes it. Errors: NULL, HIP.
 */
int qlora_workspace_set_wait_limit(void *ws, uint32_t ticks, hipStream_t stream);

/* Bytes of the quantized weight: n/2 + n/64 + 4*ceil(n/16384). */
size_t qlora_storage_bytes(int64_t d_out, int64_t d_in);

/* Bytes of the absmax-only storage (qscale == NULL): n/2 + 4*n/64, 4.5 bits per weight. */
size_t qlora_storage_bytes_absmax(int64_t d_out, int64_t d_in);

/* Workspace bytes sufficient for both qlora_forward and qlora_backward at these sizes. */
size_t qlora_workspace_bytes(int64_t d_out, int64_t d_in, int64_t T, int32_t r);

/* Host: the 16 float32 NF4 levels, ascending (c[0] = -1, c[7] = 0, c[15] = 1). */
void qlora_nf4_codebook(float out[16]);

/* Host: the 15 float32 decision thresholds (smallest float32 above each level midpoint). */
void qlora_nf4_thresholds(float out[15]);

/* Host: static text for a status code. */
const char *qlora_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */

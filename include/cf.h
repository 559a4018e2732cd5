/*
 * cf.h - C ABI of libcf: CompactFusion step-wise activation residual compression
 * with sender-side error feedback, on MI355X (gfx950).
 *
 * Method: "Accelerating Parallel Diffusion Model Serving with Residual
 * Compression" (CompactFusion summary), section Approach; the measured-effects
 * table names the variants built here (Compact-1bit, Compact-2bit,
 * Compact-Lowrank) and the warmup steps.  In short: what crosses the wire at a
 * denoising step is the residual between a layer's activation and the
 * reconstruction both sides already hold, compressed; the sender keeps the part
 * the compression lost and feeds it into the next step's residual; the low-rank
 * variant sends two INT4-quantized factors instead of codes.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a DEVICE pointer on the current HIP device, allocated and
 *     owned by the caller, who keeps it alive until the stream work is done.
 *     The library allocates nothing in these calls and keeps no pointer after
 *     a call returns.
 *   - Calls are stream-ordered and asynchronous: CF_OK means "validated and
 *     enqueued on `stream`" (a hipStream_t; NULL = the null stream).  A fault
 *     inside a kernel surfaces at the caller's next synchronisation.
 *   - Every argument is validated before anything is enqueued, so a call that
 *     returns an error has written nothing (a half-applied state update would
 *     corrupt the error feedback).
 *   - Activations `a` are bf16 (CF_BF16, raw 16-bit storage) or fp32 (CF_F32),
 *     row-major; the reconstruction `ahat` and the error buffer `err` are fp32.
 *   - The error feedback lives in `ahat`: the next step's residual is a - ahat, so
 *     the sender never reads `err`, and resuming needs `ahat` alone.  The senders
 *     therefore take `err = NULL`, which skips writing it (4 bytes per element less;
 *     the low-rank sender also skips re-reading `a`).
 *     State lives only in caller buffers, so a checkpoint is a copy of them.
 *   - A group is CF_GROUP = 128 contiguous elements; `numel` must be a positive
 *     multiple of 128, at most 2^33.  Several tensors laid out back to back may be passed as
 *     one call (one "slab"), since no group straddles two tensors when every
 *     tensor's size is a multiple of 128.
 *   - Every pointer must be 16-byte aligned, except `scales` (one float per
 *     group), which needs 4-byte alignment, and the top-k payload (see there);
 *     input and output ranges must not overlap.
 *   - Results are deterministic: no atomics, fixed reduction orders.
 *   - Calls on different streams with disjoint buffers may run concurrently.
 *   - Non-finite inputs give unspecified (but memory-safe) results.
 */
#ifndef CF_H
#define CF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: 0 on success, negative on error. */
enum {
    CF_OK = 0,
    CF_E_NULL = -1,      /* a required pointer is NULL */
    CF_E_SHAPE = -2,     /* numel / m / n / rank / batch out of range */
    CF_E_ALIGN = -3,     /* a pointer is misaligned (16 bytes; scales 4 bytes) */
    CF_E_ARG = -4,       /* bits, k, dtype, factor_bits or iters not supported */
    CF_E_ALIAS = -5,     /* an output range overlaps another operand */
    CF_E_WORKSPACE = -6, /* workspace missing or too small */
    CF_E_DEVICE = -7,    /* current device is not gfx950 */
    CF_E_HIP = -8,       /* the HIP runtime refused a launch; a call that launches several
                            kernels (cf_lowrank_compress) may then have applied part of
                            its update, so treat the state as lost (re-run the warmup) */
    CF_E_SCRATCH = -9    /* cf_lowrank_compress_noalloc: the call needs more scratch than
                            the fixed CF_NOALLOC_SCRATCH_BYTES */
};

enum { CF_BF16 = 0, CF_F32 = 1 };

/* Sender modes of cf_compress_ablation. */
enum { CF_MODE_NOEF = 1, CF_MODE_NAIVE = 2 };

#define CF_GROUP 128

/*
 * Warmup / initialisation (measured-effects table: the rows with one and with two
 * warmup steps).  During the first W steps the activation itself is sent and both
 * sides take it as their reconstruction:  ahat[i] = a[i]  and, when `err` is
 * not NULL (the sender), err[i] = 0.  The receiver passes err = NULL.
 *   a:    numel elements of `a_dtype`
 *   ahat: numel fp32 (out)      err: numel fp32 (out) or NULL
 */
int cf_init_state(int a_dtype, const void* a, float* ahat, float* err, int64_t numel,
                  void* stream);

/*
 * Sender step, Compact-1bit / Compact-2bit (Approach: residual against the
 * previous reconstruction with sender-side error feedback).  Per group g of 128
 * contiguous elements:
 *   r = a - ahat                                         (fp32)
 *   bits = 1: s = mean|r| over the group, taken exactly and rounded once to
 *             fp32 (to nearest, ties to even), so it depends on no summation order;
 *             code = (r < 0);  d = code ? -s : s
 *   bits = 2: s = max|r| / 1.5 (IEEE division);  sign = (r < 0),
 *             mag = (|r| > s);  code = sign | mag << 1;
 *             d = +-(mag ? 1.5*s : 0.5*s)   (levels {-1.5,-0.5,0.5,1.5}*s)
 *   ahat = ahat + d;   err = a - ahat        (each operation rounded once)
 *   codes: numel*bits/8 bytes, LSB first, groups back to back (16*bits bytes
 *          per group); scales: numel/128 fp32, one per group.
 *   a: in; ahat: in/out; err: out or NULL; codes, scales: out.
 */
int cf_compress(int bits, int a_dtype, const void* a, float* ahat, float* err, uint8_t* codes,
                float* scales, int64_t numel, void* stream);

/*
 * Receiver step: decodes codes/scales with exactly the sender's expression for
 * d and applies ahat = ahat + d, so the receiver's reconstruction equals the
 * sender's bit for bit (Approach: the receiver rebuilds the activation from
 * the transmitted residuals).
 *   codes, scales: in (as produced by cf_compress); ahat: in/out.
 */
int cf_decompress(int bits, const uint8_t* codes, const float* scales, float* ahat, int64_t numel,
                  void* stream);

/*
 * Receiver step with a bf16 copy for the consumer (the attention that reads the
 * reconstructed K/V): exactly cf_decompress, and then out[i] = the
 * round-to-nearest-even bf16 of the updated ahat[i].  Decoding several peers'
 * payloads is one call when their codes, scales, mirrors and outputs are laid out
 * back to back (peer p at offset p * numel_per_peer).
 *   out: numel bf16 (raw 16-bit storage), 16-byte aligned, out.
 */
int cf_decompress_bf16(int bits, const uint8_t* codes, const float* scales, float* ahat, uint16_t* out,
                       int64_t numel, void* stream);

/*
 * Ablation modes of the sender, for studies of the method's design (measured-
 * effects table: the row that adds residual compression with error feedback;
 * Surprising findings: 1-bit quantization of whole activations, without residuals,
 * fails).  Same
 * quantizer, codes and scales as cf_compress; per group:
 *   CF_MODE_NOEF:  r = a - a_prev (the raw step delta, no error feedback);
 *                  ahat = ahat + d (the receiver's mirror, which cf_decompress
 *                  reproduces); a_prev: numel of a_dtype, in.
 *   CF_MODE_NAIVE: r = a (the activation itself); ahat = d (its decoded value);
 *                  a_prev unused (may be NULL).
 * No error buffer is kept in either mode.
 */
int cf_compress_ablation(int mode, int bits, int a_dtype, const void* a, const void* a_prev, float* ahat,
                         uint8_t* codes, float* scales, int64_t numel, void* stream);

/*
 * Sender step, top-k sparsification of the residual (Limitations: sparsity is
 * the other fast compressor family beside quantization; the pages give no rule,
 * and the one built here is the following).  Per group g of 128 contiguous
 * elements:
 *   r = a - ahat                                               (fp32)
 *   keep the k elements of largest |r|, ordered by the bit pattern of |r| (the
 *   magnitude order for non-NaN values), equal magnitudes going to the lower
 *   index;  for each kept element i, in increasing i:
 *     idx[g*k + slot] = i (0..127);  vals[g*k + slot] = v = RNE bf16 of r[i];
 *     ahat[i] = ahat[i] + widen(v)
 *   err = a - ahat for all 128 elements (the dropped residuals stay in err).
 *   1 <= k <= 128 (k = 12 spends the 2-bit budget of 36 bytes per group).
 *   idx: numel/128*k bytes, any alignment; vals: numel/128*k bf16 (raw 16-bit),
 *   2-byte aligned; a, ahat, err: 16-byte aligned.
 *   a: in; ahat: in/out; err: out or NULL; idx, vals: out.
 */
int cf_topk_compress(int k, int a_dtype, const void* a, float* ahat, float* err, uint8_t* idx, uint16_t* vals,
                     int64_t numel, void* stream);

/*
 * Receiver step, top-k: ahat[g*128 + (idx[g*k+s] & 127)] += widen(vals[g*k+s]) for
 * every slot s, the sender's own update, so the reconstructions agree bit for bit.
 * Only the low 7 bits of an index byte are used, so any payload stays inside its
 * group; a payload that repeats an index within a group (the sender never does)
 * gives an unspecified value at that element.
 *   idx, vals: in (as produced by cf_topk_compress); ahat: in/out, 16-byte aligned.
 */
int cf_topk_decompress(int k, const uint8_t* idx, const uint16_t* vals, float* ahat, int64_t numel,
                       void* stream);

/*
 * Sender step, Compact-Lowrank (Approach: low-rank compression of the residual
 * with INT4 quantization of the factors; Key results: rank 32 with INT4 factors
 * gives about 100x; measured-effects table: 2 vs 10 subspace iterations;
 * Experimental setup, "Builds on": PowerSGD-style subspace iteration).
 * `batch` tensors of m x n (row-major) laid out back to back.  Per tensor:
 *   r = a - ahat;  Q = q_state;
 *   repeat `iters` times:  Y = r Q;  P = orth(Y);  Q = r^T P
 *     orth: thin QR factor with diag(R) >= 0; a rank-deficient column (|R_jj| <=
 *     1e-5 ||Y||_F) gives a zero column of P;
 *   factor_bits 4:  U = int4(P), V = int4(Q): per column j, s_j = max|x| / 7,
 *     code = rint(x / s_j) clamped to [-7, 7] (0 when s_j = 0), two's-complement
 *     nibbles, row-major rows x rank, low nibble first;  U^ = code * s_j;
 *   factor_bits 16: U, V = the round-to-nearest-even bf16 of P, Q, row-major
 *     (rows x rank) (the table's "Pure Lowrank" variant); scales unused;
 *   factor_bits 32: U = P, V = Q as fp32 row-major (rows x rank); scales unused;
 *   ahat = ahat + U^ V^^T;   err = a - ahat;
 *   q_state = Q (a column zeroed by the rank guard keeps its previous value).
 * Buffers (all device memory):
 *   a: batch*m*n (a_dtype), in; ahat: batch*m*n fp32, in/out; err: out or NULL;
 *   q_state: batch*n*rank fp32, in/out (the start basis; a seeded N(0,1) matrix
 *     before the first compressed step);
 *   u: batch*m*rank*factor_bits/8 bytes, out; v: batch*n*rank*factor_bits/8 bytes,
 *     out; both 4-byte aligned;
 *   u_scales, v_scales: batch*rank fp32, out (may be NULL unless factor_bits = 4);
 *   workspace: ws_bytes >= cf_lowrank_workspace_bytes(m, n, rank, batch), 256-byte
 *     aligned; scratch, its contents are not preserved between calls.
 * Limits: m and n positive multiples of 16; batch*m*n <= 2^33; 1 <= rank <=
 *   min(m, n, 64); rank even when factor_bits = 4; 1 <= iters <= 64; batch >= 1;
 *   every kernel grid within a dispatch's 2^32 - 1 work-items (only extreme shapes,
 *   such as a single row block of 2^28 columns, reach that); CF_E_SHAPE otherwise.
 *   a, ahat, err 16-byte aligned; the other pointers 4-byte aligned.
 * Arithmetic is fp32 (fp64 inside orth).  Results are deterministic for given shapes,
 * rank, iters and batch; a tensor's last bits depend on the batch it is sent in, since
 * the fp32 sums of Y follow the work's split of the whole batch into equal parts.
 */
int cf_lowrank_compress(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                        int rank, int iters, int factor_bits, int batch, float* q_state, void* u,
                        float* u_scales, void* v, float* v_scales, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * Receiver step, Compact-Lowrank (Approach: the receiver rebuilds the activation by
 * adding the decoded low-rank residual to its copy of the previous reconstruction;
 * measured-effects table: rank 32 with INT4 factors):  ahat = ahat + U^ V^^T for
 * `batch` tensors, with the sender's dequantization and the sender's reconstruction
 * kernel, so the receiver's ahat equals the sender's bit for bit.  Buffers and limits
 * as in cf_lowrank_compress; u, u_scales, v, v_scales in; ahat in/out.
 */
int cf_lowrank_decompress(int factor_bits, const void* u, const float* u_scales, const void* v,
                          const float* v_scales, float* ahat, int64_t m, int64_t n, int rank,
                          int batch, void* stream);

/*
 * cf_lowrank_compress without a workspace argument, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Identical arguments, results and errors to
 * cf_lowrank_compress, except that the workspace is a fixed buffer of
 * CF_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory from the first
 * load of its code object until the process ends; the call allocates nothing.
 *   - A call whose cf_lowrank_workspace_bytes(m, n, rank, batch) exceeds
 *     CF_NOALLOC_SCRATCH_BYTES returns CF_E_SCRATCH and writes nothing (64 MiB holds
 *     four 1024 x 3072 tensors at rank 32; split larger batches into several calls).
 *   - Every call on one GPU uses that GPU's one buffer: calls that may overlap in time
 *     on one GPU (different streams, or several host threads) race and give wrong
 *     results.  Order them on one stream, or use cf_lowrank_compress with a workspace
 *     per stream.  Nothing in the buffer needs to start at zero: each call writes every
 *     byte it reads before reading it.
 */
#define CF_NOALLOC_SCRATCH_BYTES (64u << 20)

int cf_lowrank_compress_noalloc(int a_dtype, const void* a, float* ahat, float* err, int64_t m, int64_t n,
                                int rank, int iters, int factor_bits, int batch, float* q_state, void* u,
                                float* u_scales, void* v, float* v_scales, void* stream);

/* Workspace bytes cf_lowrank_compress needs (0 for arguments outside the limits). */
size_t cf_lowrank_workspace_bytes(int64_t m, int64_t n, int rank, int batch);

/* Bytes of packed codes for numel elements at `bits` per element (numel*bits/8),
 * or a negative status for invalid arguments. */
int64_t cf_codes_bytes(int64_t numel, int bits);

/* Human-readable name of a status code (static storage). */
const char* cf_strerror(int status);

/* ABI version of this header: 1. */
int cf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CF_H */

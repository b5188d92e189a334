/*
 * hqml -- batched state-vector training step of a hardware-efficient ansatz
 * on AMD Instinct MI355X (gfx950), with gate fusion in the forward pass and in
 * the adjoint backward pass.
 *
 * The operation (Kawase, "Fast and memory-efficient classical simulation of
 * quantum machine learning via forward and backward gate fusion",
 * arXiv:2603.02804; hugo-pages summary, sections 1.2 and 2.1):
 *   per sample b, psi_0 = prod_q Ry(x[b][q]) |0...0>; then L layers, each
 *   applying Rx(theta[l][q][0]), Ry(theta[l][q][1]), Rz(theta[l][q][2]) to every
 *   qubit q followed by CZ(q, q+1) for q = 0..n-2; R_s(t) = exp(-i t s/2);
 *   qubit q is bit q of the amplitude index.  E_b = <psi_M|O|psi_M> with
 *   O = Z_0 by default, or any Pauli string: Z on the qubits of obs_mask only,
 *   X on those of obs_x_mask only and Y on those in both masks.
 *   The gradient is the adjoint-method gradient of section 1.2:
 *   dL/dtheta_j = Re<lambda_j| dU_j/dtheta_j |psi_{j-1}>, lambda_{j-1} = U_j^dag lambda_j,
 *   seeded with lambda_M = 2 (dL/dE_b) O psi_M, summed over the batch.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to contiguous row-major fp32
 *     arrays owned by the caller; the library never frees or keeps them.
 *     x: [B][n] encoding angles; theta: [L][n][3] (Rx, Ry, Rz angle of qubit q
 *     in layer l); y: [B] labels; expz: [B]; loss: [1]; grad: [L][n][3];
 *     dL_dE: [B].  Each array must be device memory of the context's device
 *     (pinned host memory mapped into it also works) and fit inside the HIP
 *     allocation that holds it; otherwise the call returns HQML_ERR_ARG before
 *     queuing anything (a NULL, pageable-host or too-short array).  The range
 *     check sees the runtime's allocation, not a caller's sub-allocation: a
 *     tensor inside a larger segment of a caching allocator is checked against
 *     the end of that segment.  A pointer that passed is remembered per
 *     argument with its allocation's base and size; a repeat call re-reads
 *     only the allocation range.
 *   - Work is queued on the context's stream and is asynchronous: outputs are
 *     valid once that stream has synchronised.  Argument errors are detected
 *     on the host before anything is queued.
 *   - Return value: HQML_OK or a negative hqml_status.  On error, outputs are
 *     unspecified, nothing leaks, and hqml_last_error(ctx) describes it.
 *     No entry point aborts or throws across the ABI.
 *   - Results are bitwise reproducible: every reduction has a fixed order and
 *     no floating-point atomics are used.
 *   - A context is used by one host thread at a time; distinct contexts are
 *     independent.
 */
#ifndef HQML_H
#define HQML_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hqml_ctx hqml_ctx;

typedef enum {
    HQML_OK = 0,
    HQML_ERR_ARG = -1,          /* invalid argument (null pointer, size out of range) */
    HQML_ERR_OOM = -2,          /* device memory could not be reserved */
    HQML_ERR_HIP = -3,          /* a HIP runtime call or kernel launch failed */
    HQML_ERR_STATE = -4,        /* call out of order (e.g. backward without a saved forward) */
    HQML_ERR_UNSUPPORTED = -5   /* valid request the library does not implement */
} hqml_status;

typedef enum {
    HQML_STORE_FP32 = 0,        /* saved states as complex fp32 (8 bytes per amplitude) */
    HQML_STORE_BF16 = 1,        /* saved states as bf16 (re, im) pairs, round to nearest even;
                                   arithmetic stays fp32 (the pages' mem-save mode, section 2.3) */
    HQML_STORE_FP64 = 2         /* saved states as complex fp64 (16 bytes per amplitude);
                                   needs HQML_COMPUTE_FP64 (full complex128 mode) */
} hqml_storage;

typedef enum {
    HQML_COMPUTE_FP32 = 0,      /* arithmetic, lambda and partial sums in fp32 (fp64 reductions) */
    HQML_COMPUTE_FP64 = 1       /* arithmetic, lambda and partial sums in fp64, with fp32 or fp64
                                   saved states (the pages' higher-precision modes; n_qubits 13
                                   is not supported in this mode) */
} hqml_compute;

typedef enum {
    HQML_FUSED = 0,             /* fused forward and adjoint passes (the method itself) */
    HQML_GATE_BY_GATE = 1       /* comparator without fusion: one kernel per gate in the forward
                                   pass and per gate in the adjoint pass, which un-computes psi
                                   gate by gate (sections 2.1-2.2 compare the two); fp32 states
                                   only, no checkpointing */
} hqml_fusion;

typedef enum {
    HQML_ENT_CZ = 0,            /* every layer ends with CZ(q, q+1), q = 0..n-2 (section 2.1) */
    HQML_ENT_CNOT = 1           /* every layer ends with CNOT(q, q+1) (control q, target q+1) for
                                   q = 0, 1, ..., n-2 in that order, a permutation of the amplitude
                                   indices (section 3.2 fuses CNOTs by recomputing indices).  With
                                   n_qubits <= 13 the index map is applied in local memory; with
                                   n_qubits >= 14 it mixes every index bit, so the fused passes run
                                   one per qubit group and layer (twice the CZ chain's state traffic
                                   at 20 qubits) and read each layer's input through the map; they
                                   measure the string conjugated by the last chain, whose X/Y part
                                   covers qubits q and q+1 for each X/Y factor on q (the limit of 9
                                   such qubits above qubit 3 applies to it).  The HQML_GATE_BY_GATE
                                   comparator applies one kernel per CNOT at any width */
} hqml_entangler;

typedef struct {
    int n_qubits;      /* 1..29 */
    int n_layers;      /* >= 1 */
    int max_batch;     /* >= 1; workspaces are sized for this many samples */
    int storage;       /* hqml_storage */
    int ckpt_block;    /* 0: keep every fused-pass output for the backward pass;
                          b > 0: keep only one state every b layers and recompute the
                          block's forward passes during the backward pass
                          (gradient checkpointing, section 2.3) */
    int device;        /* HIP device ordinal */
    void *stream;      /* hipStream_t to queue work on; NULL = the null stream */
    int fusion;        /* hqml_fusion; 0 = HQML_FUSED */
    int compute;       /* hqml_compute; 0 = HQML_COMPUTE_FP32 */
    int obs_mask;      /* observable O, a Pauli string (the general O of section 1.2 restricted
                          to tensor products of I, X, Y, Z): qubit q (bit q) carries Z if only
                          obs_mask has it, X if only obs_x_mask has it, Y if both do, I if
                          neither.  Both 0 = Z on qubit 0 (the default).  Only qubits
                          0..n_qubits-1.  With X/Y factors and n_qubits >= 14, at most 9 of
                          them may sit on qubits >= 4 (they must fit one tile view) */
    int obs_x_mask;
    int entangler;     /* hqml_entangler; 0 = HQML_ENT_CZ */
} hqml_config;

/* Device bytes hqml_create would reserve for cfg.  Host-only: makes no HIP call.
 * Returns 0 for an invalid cfg. */
size_t hqml_workspace_bytes(const hqml_config *cfg);

/* Validate cfg, reserve every device workspace once, and return a context in
 * *out.  HQML_ERR_OOM if the workspace exceeds the device's free memory (checked
 * before any allocation) or an allocation fails.  Nothing is allocated later. */
int hqml_create(const hqml_config *cfg, hqml_ctx **out);

/* Release the context and its workspaces (waits for its stream).  NULL is a no-op. */
int hqml_destroy(hqml_ctx *ctx);

/* Forward pass for B samples (0 <= B <= max_batch): expz[b] = <O> of sample b.
 * save_for_backward != 0 keeps what hqml_backward needs (the fused-pass outputs,
 * or checkpoints) until the next forward on this context.  B == 0 queues nothing. */
int hqml_forward(hqml_ctx *ctx, int B, const float *x, const float *theta, float *expz,
                 int save_for_backward);

/* Adjoint backward pass for the batch of the last hqml_forward(..., 1) on this
 * context: grad[l][q][a] = sum_b dL_dE[b] * dE_b/dtheta[l][q][a] (fp64 reduction,
 * stored as fp32).  HQML_ERR_STATE if no forward was saved; theta and x are the
 * ones that forward saw.  Fused contexts keep the saved forward, so several
 * backward calls may follow one forward; a HQML_GATE_BY_GATE context un-computes
 * its one saved state in place, so each backward needs a new saved forward. */
int hqml_backward(hqml_ctx *ctx, const float *dL_dE, float *grad);

/* One training step with the mean-squared-error loss on <O> (the pages' training
 * objective; mean over the batch): expz = E_b, loss = (1/B) sum_b (E_b - y_b)^2,
 * grad = dloss/dtheta.  1 <= B <= max_batch.  Equivalent to forward + backward with
 * dL_dE[b] = 2 (E_b - y_b) / B, with the last fused pass of the forward sweep and the
 * first of the backward sweep run as one kernel. */
int hqml_train_step(hqml_ctx *ctx, int B, const float *x, const float *theta, const float *y,
                    float *expz, float *loss, float *grad);

/* The same three calls with fp64 arrays (x, theta, y, dL_dE in; expz, loss, grad out),
 * for contexts whose results are wanted in fp64 (normally HQML_COMPUTE_FP64; any fused
 * context accepts them).  HQML_ERR_UNSUPPORTED on a HQML_GATE_BY_GATE context. */
int hqml_forward_f64(hqml_ctx *ctx, int B, const double *x, const double *theta, double *expz,
                     int save_for_backward);
int hqml_backward_f64(hqml_ctx *ctx, const double *dL_dE, double *grad);
int hqml_train_step_f64(hqml_ctx *ctx, int B, const double *x, const double *theta, const double *y,
                        double *expz, double *loss, double *grad);

/* Allocation-free training step, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * computes exactly what hqml_train_step computes on a context created from *cfg (same
 * kernels, same order, bitwise the same results), for the fused whole-circuit sizes only
 * (n_qubits <= 13), and needs no context.  The caller passes inputs and outputs as for
 * hqml_train_step (fp32 device arrays of cfg->device; 1 <= B <= cfg->max_batch); work is
 * queued on cfg->stream.  Every intermediate (rotation tables, per-sample gradient
 * statistics, sums) lives in one library-owned device buffer of
 * HQML_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library's code is loaded on that
 * GPU and held until the process ends; the call allocates nothing.  A step needs
 * 24 B per sample, layer and qubit (fp64 statistics), 145 B (fp32 compute) or 169 B
 * (fp64 compute) per layer and qubit (tables), 16 B or 32 B per sample and qubit plus
 * 24 B per sample, each of its ten parts rounded up to 256 B; a batch beyond the buffer
 * returns HQML_ERR_ARG.  HQML_ERR_UNSUPPORTED for n_qubits > 13 or
 * HQML_GATE_BY_GATE.  Errors are reported by hqml_last_error(NULL).
 * All calls on one GPU share its buffer, which keeps the last call's contents: calls
 * that overlap on one GPU (from two host threads, or queued on two streams whose work
 * runs concurrently) race and give wrong results. */
#define HQML_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int hqml_train_step_noalloc(const hqml_config *cfg, int B, const float *x, const float *theta,
                            const float *y, float *expz, float *loss, float *grad);

/* Static text for a status code. */
const char *hqml_status_str(int status);

/* Text of the last error on ctx ("" if none); with ctx == NULL, the last error of
 * hqml_create or hqml_train_step_noalloc on this thread. */
const char *hqml_last_error(const hqml_ctx *ctx);

/* ---- instrumentation (benchmarking; not needed for training) ---- */

/* Kernel families timed by hqml_kernel_times. */
typedef enum {
    HQML_K_FWD_PASS = 0,    /* fused forward tile pass (one per fused block) */
    HQML_K_BWD_PASS = 1,    /* fused adjoint tile pass (one per fused block) */
    HQML_K_SMALL = 2,       /* whole-circuit kernel for n <= 13 */
    HQML_K_OTHER = 3,       /* table preparation and reductions */
    HQML_K_GATE = 4,        /* one gate of a HQML_GATE_BY_GATE context (forward or adjoint) */
    HQML_K_COUNT = 5
} hqml_kernel_kind;

/* Enable (1) or disable (0) per-launch HIP event timing on ctx's stream.  While
 * enabled, every kernel launch is bracketed by a pair of HIP events. */
int hqml_set_timing(hqml_ctx *ctx, int enable);

/* Synchronise ctx's stream and report, per hqml_kernel_kind, the summed event time
 * in milliseconds (ms[HQML_K_COUNT]) and the number of launches (count[HQML_K_COUNT])
 * since timing was enabled or last reset; reset != 0 clears the counters. */
int hqml_kernel_times(hqml_ctx *ctx, double *ms, long long *count, int reset);

/* Number of batch chunks a training step on the tile path (n >= 14) pipelines: chunk
 * k+1's forward sweep runs on a second stream of the context while chunk k's adjoint
 * sweep runs on the context's stream.  Samples are independent, so results are
 * bitwise the same for every chunk count.  0 = automatic (2 when ckpt_block > 0, else
 * 1), 1 = no overlap, at most 8; a chunk keeps at least 256 tiles.  Per-launch timing
 * (hqml_set_timing) also disables the overlap. */
int hqml_set_overlap(hqml_ctx *ctx, int chunks);

/* Plan facts for reporting: fused forward passes per training step, backward
 * passes per training step, tile workgroups per pass, bytes of state per sample.
 * For a HQML_GATE_BY_GATE context: forward gate kernels, adjoint gate kernels and
 * workgroups per sample of one gate kernel. */
int hqml_plan_info(const hqml_ctx *ctx, int *fwd_passes, int *bwd_passes,
                   int *tiles_per_sample, size_t *state_bytes);

/* JSON description of the fused-pass schedule hqml_create would use for cfg (views,
 * passes, where each layer's gradient statistics are formed).  Host-only.  Writes at
 * most len bytes including the terminating NUL and returns the full length needed
 * (excluding the NUL), or a negative hqml_status for an invalid cfg. */
long long hqml_describe_plan(const hqml_config *cfg, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* HQML_H */

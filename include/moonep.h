/*
 * moonep.h -- C ABI of libmoonep.so: the balanced expert-parallel hot path of
 * MoonEP (redundant-expert planning, zero-copy permute/unpermute, grouped
 * SwiGLU expert GEMM, replica gradient reduction) on one AMD Instinct MI355X
 * (gfx950).
 *
 * Pages cited (title, site):
 *   [AT] "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert Parallelism
 *        Library for MoE Training", aitrending.vip
 *   [AL] "MoonshotAI/MoonEP", agentlenshq.com
 *   [TD] "MoonEP balances AI experts in MoE models ...", twodots.gr
 *   [TC] "The Busiest Rank Sets Your Step Time: Running MoonEP's Planning Code
 *        Ourselves", thakicloud.com
 *
 * Model.  R expert-parallel ranks are emulated as R static partitions of one
 * GPU's memory.  Rank r holds S tokens; each token routes to K distinct experts
 * out of E; rank r is the home of experts [r*E/R, (r+1)*E/R).  Every rank serves
 * exactly C = S*K (token, k) rows after planning [TD, summary; TC, Overview].
 * The weight tensor of a projection has rows [0, E) = home experts and rows
 * [E, E+B) = the rank's B prefetch slots [TD, memory contract; TC, Installation
 * and integration].  Here the home rows live in one [E, ...] array and the
 * slot rows of all ranks in one [R, B, ...] array.
 *
 * Conventions for every entry point.
 *   - Pointers are device pointers unless stated otherwise; the caller owns and
 *     allocates every buffer; the library allocates nothing and keeps no state
 *     between calls besides loaded kernels.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; nothing synchronises the host (the
 *     static shapes make that possible [TD, architecture; TC, "What the
 *     technique is"]).
 *   - Layouts are dense row-major.  bf16 tensors are raw 16-bit bfloat16.
 *   - Return value: MOONEP_OK, or a negative code detected on the host before
 *     anything is enqueued (bad dims, NULL or misaligned pointer), or
 *     MOONEP_EHIP if a launch failed.  Problems in the routing data itself are
 *     found on the device and reported in stats[0] (bits MOONEP_ST_*), with no
 *     host synchronisation.
 *   - Device pointers must be 16-byte aligned; row sizes (H and I elements)
 *     must be multiples of 8.
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moonep_dims {
    int32_t R;       /* emulated EP ranks, 1..64                                   */
    int32_t E;       /* routed experts, multiple of R, E/R <= 64, E <= 1024         */
    int32_t B;       /* prefetch slots per rank, 0..64                              */
    int32_t S;       /* tokens per rank, >= 1                                       */
    int32_t K;       /* experts per token, 1..min(E, 16)                            */
    int32_t H;       /* hidden size, multiple of 8                                  */
    int32_t I;       /* SwiGLU intermediate size, multiple of 8 (0 if no expert FFN) */
    uint32_t flags;  /* MOONEP_TRAINING | MOONEP_F32_ROWS | MOONEP_GRAD_ACCUM | phases */
} moonep_dims_t;

#define MOONEP_TRAINING 1u   /* plan for training: a fallback replica sets MOONEP_ST_TRAIN_FALLBACK */
#define MOONEP_F32_ROWS 2u   /* dispatch/combine rows are float32 instead of bf16 */
#define MOONEP_GRAD_ACCUM 4u /* grouped_ffn_backward adds into dw*_home / dw*_red instead of writing them */
/* moonep_plan / moonep_plan_noalloc: the low-migration rule instead of the default chain.  Both
 * keep exactly S*K rows and at most one remote home group per rank; this one moves fewer rows
 * under strong skew ([TC, What we measured, Table 1] "migrated tokens"), e.g. 38.1% instead of
 * 44.2% of all rows at the lognormal sigma = 5 workload, where the exact minimum is 38.1%. */
#define MOONEP_PLAN_LOWMIG 512u

/* Phase selection for the expert FFN calls.  Each phase is one GEMM kernel.  A call runs the
 * phases of its own that are set in flags, in the order listed; with none of its phases set it
 * runs all of them.  Bits of the other call are ignored.  Running phases in separate calls
 * gives the same results as one call, provided the inputs a phase reads (noted) are in place:
 * e.g. the weight-gradient phases may be deferred to overlap other work. */
#define MOONEP_PHASE_GATE_UP 8u   /* grouped_ffn: [Gt U] = X W13, act = silu(Gt) U, gu_save  */
#define MOONEP_PHASE_DOWN 16u     /* grouped_ffn: y = act W2 (reads act)                      */
#define MOONEP_PHASE_DACT 32u     /* backward: dA = dY W2^T and SwiGLU' -> dGt|dU in gu_save  */
#define MOONEP_PHASE_DX 64u       /* backward: drecv = [dGt dU] W13^T (reads dGt|dU)          */
#define MOONEP_PHASE_DW2 128u     /* backward: dW2 = A^T dY                                   */
#define MOONEP_PHASE_DW13 256u    /* backward: dW13 = X^T [dGt dU] (reads dGt|dU)             */

enum {
    MOONEP_OK = 0,
    MOONEP_EINVAL = -1,   /* bad dims or NULL pointer       */
    MOONEP_EALIGN = -2,   /* pointer not 16-byte aligned    */
    MOONEP_EHIP = -3,     /* a HIP launch failed            */
    MOONEP_ENOTSUP = -4,  /* combination not supported      */
    MOONEP_ETOOBIG = -5   /* dims need a larger plan workspace than moonep_plan_noalloc holds */
};

/* Device-detected routing problems, OR-ed into stats[0]. */
#define MOONEP_ST_BAD_ID 1          /* an expert id outside [0, E): no plan made        */
#define MOONEP_ST_DUP_ID 2          /* a token names one expert twice: no plan made     */
#define MOONEP_ST_CAPACITY 4        /* some rank does not total S*K rows (never for a valid plan) */
#define MOONEP_ST_OVERFLOW 8        /* plan entry table overflow (never for a valid plan)         */
#define MOONEP_ST_TRAIN_FALLBACK 16 /* training plan has replicas beyond the B slots (informational) */

/* stats[16] int32 written by moonep_plan:
 *  0 status bits            1 replicas (plan entries)   2 replicas in prefetch slots
 *  3 fallback replicas      4 fallback rows             5 migrated rows (sum of replica rows)
 *  6 migration lower bound: sum over ranks of max(0, P[q] - S*K)
 *  7 max per-expert load    8 max rows routed to one home rank (before planning)
 *  9 min rows routed to one home rank   10 donor ranks   11 receiver ranks
 * 12 max replicas on one rank           13 total planned rows (= R*S*K)   14, 15 zero
 * Replicas are [TC, What we measured, Table 1]'s "copy slots"; migrated rows its
 * "migrated tokens". */
#define MOONEP_NSTATS 16

/* Bytes of the opaque device workspace that moonep_plan fills and the other
 * entry points read.  Pure host function.  Returns 0 for invalid dims. */
size_t moonep_plan_workspace_bytes(const moonep_dims_t* dims);

/* Online redundant-expert planning [TC, "What the technique is" flowchart:
 * router output -> planning kernel; AL, How it works; TD, memory contract].
 *   topk       [R, S, K] int32  expert ids chosen by the router for each token (k order kept)
 *   plan_ws    workspace of moonep_plan_workspace_bytes() bytes; stays valid (and is read by
 *              prefetch / grouped_ffn / reduce_grad) until the next moonep_plan on it.
 *              grouped_ffn and grouped_ffn_backward also use words of it as tile counters
 *              (reset on the stream before each GEMM phase), so FFN calls on one workspace
 *              must not run concurrently.
 *   cu_seqlens [R, E+B+1] int32 out: per rank, prefix sums of the rows served by each weight
 *              row (home rows [0,E), slot rows [E,E+B)); cu_seqlens[q][E+B] == S*K
 *   dest       [R, S, K] int32 out: absolute row in the [R*S*K] receive buffer where the
 *              (token, k) row goes, computed on the send side (zero-copy permute
 *              [TC, "What the technique is"]); -1 when no plan was made
 *   stats      [16] int32 out (see above)
 * The plan follows a fixed deterministic rule (each rank's duplicates come from at most one
 * other rank's home group [TC, Installation and integration]; replicas beyond the B slots
 * read the home row, "fallback" [TD, memory contract]); results are bit-identical run to run. */
int moonep_plan(const moonep_dims_t* dims, const int32_t* topk, void* plan_ws,
                int32_t* cu_seqlens, int32_t* dest, int32_t* stats, void* stream);

/* moonep_plan for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same rule and the same cu_seqlens, dest
 * and stats, bit for bit, as moonep_plan; the plan workspace is a static device array of the
 * library, MOONEP_NOALLOC_WS_BYTES on every GPU the library runs on, held until the process
 * ends.  It calls no allocator.  Its output serves the plan + dispatch + combine path (dest,
 * cu_seqlens); prefetch, grouped_ffn and reduce_grad read a caller-owned moonep_plan workspace.
 *   topk, cu_seqlens, dest, stats  as for moonep_plan
 * Returns MOONEP_ETOOBIG (nothing enqueued) when moonep_plan_workspace_bytes(dims) exceeds
 * MOONEP_NOALLOC_WS_BYTES (8 MiB: e.g. R=8, E=256, S=4096, K=8 needs 2.1 MB; R=8, E=384,
 * S=8192, K=8 about 5.7 MB), MOONEP_EHIP if the array's device address cannot be obtained.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (other streams,
 * other host threads) race and must be serialised by the caller. */
#define MOONEP_NOALLOC_WS_BYTES (8u << 20)
int moonep_plan_noalloc(const moonep_dims_t* dims, const int32_t* topk, int32_t* cu_seqlens,
                        int32_t* dest, int32_t* stats, void* stream);

/* Weight prefetch [TC, flowchart "Weight prefetch"; TD, memory contract]: for every replica
 * that got slot j on rank q, copy the home expert's weights into that slot.
 *   w13_home [E, H, 2I] bf16 (gate | up columns), w2_home [E, I, H] bf16
 *   w13_slot [R, B, H, 2I] bf16 out, w2_slot [R, B, I, H] bf16 out (unused slots untouched) */
int moonep_prefetch(const moonep_dims_t* dims, const void* plan_ws,
                    const void* w13_home, const void* w2_home,
                    void* w13_slot, void* w2_slot, void* stream);

/* Fused zero-copy permute [TC, "What the technique is"; AL, How it works; TD, architecture]:
 * recv[dest[r,s,k]] = src[r,s] for every (token, k).
 *   src  [R, S, H] bf16 (float32 with MOONEP_F32_ROWS)
 *   row_scale [R, S, K] float32 or NULL.  NULL: bitwise copy.  Otherwise each copy is
 *        multiplied by its scale in float32 and rounded to nearest even (the backward of a
 *        gate-weighted combine).
 *   recv [R*S*K, H] out, same element type as src.  Rows whose dest is -1 are skipped. */
int moonep_dispatch(const moonep_dims_t* dims, const int32_t* dest, const void* src,
                    const float* row_scale, void* recv, void* stream);

/* Fused unpermute [TC, flowchart "combine"]: out[r,s] = sum over k (in k order, float32
 * accumulation) of gates[r,s,k] * y[dest[r,s,k]], rounded to nearest even.
 *   y     [R*S*K, H] bf16 (float32 with MOONEP_F32_ROWS)
 *   gates [R, S, K] float32, or NULL for unit weights (the backward of dispatch)
 *   out   [R, S, H] out, same element type as y. */
int moonep_combine(const moonep_dims_t* dims, const int32_t* dest, const void* y,
                   const float* gates, void* out, void* stream);

/* Staged (not zero-copy) permute and unpermute, the baseline that measures what sender-side
 * final positions save [TC, "What the technique is"; AT, Technical Details; AL, Highlights]:
 * rows first land in arrival order, stage[(r, s, k)] = scale(src[r, s]), and a separate
 * sort-copy then moves them to their expert-grouped rows, recv[dest[p]] = stage[p].  Combine
 * mirrors it: stage[p] = y[dest[p]], then out[r, s] = sum over k of gates * stage[(r, s, k)].
 * Results are bit-identical to moonep_dispatch / moonep_combine; every row crosses HBM twice more.
 *   stage [R*S*K, H] scratch of the row type (contents on return: the arrival-order rows)
 *   other arguments as for moonep_dispatch / moonep_combine. */
int moonep_dispatch_staged(const moonep_dims_t* dims, const int32_t* dest, const void* src,
                           const float* row_scale, void* stage, void* recv, void* stream);
int moonep_combine_staged(const moonep_dims_t* dims, const int32_t* dest, const void* y,
                          const float* gates, void* stage, void* out, void* stream);

/* Grouped SwiGLU expert FFN over the receive buffer [TC, flowchart "Group GEMM"; TD, memory
 * contract: cu_seqlens selects the active weight rows].  For each group (rank q, weight row w)
 * with rows X_g:  [Gt U] = X_g W13[w];  A = silu(Gt) * U;  Y_g = A W2[w]; bf16 inputs, float32
 * accumulation, bf16 outputs.  Weight row w < E reads w13_home/w2_home[w] (home expert, or a
 * fallback replica reading the home row); w >= E reads slot (q, w-E).
 *   recv    [R*S*K, H] bf16
 *   gu_save [R*S*K, 2I] bf16 out (Gt | U, kept for the backward) or NULL
 *   act     [R*S*K, I] bf16 out
 *   y       [R*S*K, H] bf16 out
 * Phases (flags): MOONEP_PHASE_GATE_UP, MOONEP_PHASE_DOWN. */
int moonep_grouped_ffn(const moonep_dims_t* dims, const void* plan_ws, const int32_t* cu_seqlens,
                       const void* recv, const void* w13_home, const void* w2_home,
                       const void* w13_slot, const void* w2_slot,
                       void* gu_save, void* act, void* y, void* stream);

/* Backward of moonep_grouped_ffn.  dA = dY W2^T; dGt = dA U sig(Gt)(1 + Gt(1 - sig(Gt)));
 * dU = dA silu(Gt); dX = [dGt dU] W13^T; dW2 = A^T dY; dW13 = X^T [dGt dU].
 * Weight gradients of slot replicas go to the separate fp32 reduce buffers (they must not
 * reach the framework's gradient reduction [TD, memory contract; AT, Technical Details]);
 * home experts' gradients go to dw*_home.  A fallback replica (training with B < E/R, an
 * extension: the pages ask for B = E/R in training) contributes to its home expert's gradient
 * together with the home rows.
 *   dy        [R*S*K, H] bf16 upstream gradient of y (e.g. moonep_dispatch with row_scale)
 *   gu_save   in: Gt|U from moonep_grouped_ffn; out: overwritten with dGt|dU
 *   drecv     [R*S*K, H] bf16 out
 *   dw13_home [E, H, 2I] float32, dw2_home [E, I, H] float32: every expert's gradient of this call
 *   dw13_red  [R, B, H, 2I] float32, dw2_red [R, B, I, H] float32: the gradient of each slot
 *             replica of this call (slots without a replica are untouched)
 *   Without MOONEP_GRAD_ACCUM the gradients are written (each home expert, including experts
 *   that received no rows, and each used slot); with it they are added to what the buffers
 *   hold (e.g. accumulation over micro-batches; the reduce slots are zero after
 *   moonep_reduce_grad).
 * Phases (flags): MOONEP_PHASE_DACT, MOONEP_PHASE_DX, MOONEP_PHASE_DW2, MOONEP_PHASE_DW13.
 * gu_save holds Gt|U until MOONEP_PHASE_DACT has run and dGt|dU afterwards.  The
 * GEMM phases use tile counters in plan_ws: FFN calls on one plan_ws must not overlap. */
int moonep_grouped_ffn_backward(const moonep_dims_t* dims, const void* plan_ws,
                                const int32_t* cu_seqlens, const void* recv,
                                const void* gu_save, const void* act, const void* dy,
                                const void* w13_home, const void* w2_home,
                                const void* w13_slot, const void* w2_slot,
                                void* drecv, float* dw13_home, float* dw2_home,
                                float* dw13_red, float* dw2_red, void* stream);

/* reduce_grad [TD, memory contract; AT, Technical Details]: for every expert, add its slot
 * replicas' reduce-buffer gradients (in replica creation order) into the home gradient, then
 * zero those slots for the next micro-batch.  Float32, in place. */
int moonep_reduce_grad(const moonep_dims_t* dims, const void* plan_ws,
                       float* dw13_home, float* dw2_home, float* dw13_red, float* dw2_red,
                       void* stream);

/* Static description of an error code. */
const char* moonep_strerror(int code);

/* Library version string. */
const char* moonep_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOONEP_H */

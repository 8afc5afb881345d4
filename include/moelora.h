/*
 * moelora.h — C ABI of the fused MoE + multi-LoRA layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (page "vLLM MoE LoRA SageMaker Bedrock", sections "Entendendo os Modelos MoE" and
 * "O Papel da Multi-LoRA"; page "Punica: Multi-Tenant LoRA Serving", proposed-method section):
 * each token is routed to its top-k experts; every selected expert applies a frozen gate_up
 * projection, SiLU-and-mul and a frozen down projection, and both projections also apply the
 * token's own LoRA adapter (shrink z = xA to rank r, expand z B added to the base output).
 * The expert outputs are combined with the router weights.
 *
 * Conventions fixed by this library where the pages are silent:
 *   - routing weights: softmax over the k selected logits; ties go to the lower expert id;
 *     slots are in descending logit order;
 *   - W1 rows 0..I-1 are gate, I..2I-1 up; act = silu(gate) * up; LoRA scale 1;
 *   - one (A1, B1) pair per (adapter, expert) for gate_up, one (A2, B2) for down;
 *   - adapter id -1 means "no adapter" for that token.
 *
 * Stored layouts ("out x in", the reduction dimension contiguous; the pages' math matrices
 * are the transposes). All tensors are dense, row-major, device memory:
 *   x            bf16 [T][h]
 *   router_logits f32 [T][E]
 *   W1           bf16 [E][2I][h]        W2  bf16 [E][h][I]
 *   A1           bf16 [nA][E][r][h]     B1  bf16 [nA][E][2I][r]
 *   A2           bf16 [nA][E][r][I]     B2  bf16 [nA][E][h][r]
 *   adapter_ids  int32 [T], each in [-1, nA)
 *   y            bf16 [T][h]  (written, not accumulated)
 *
 * Ownership and ordering: the caller owns every buffer (inputs, outputs, workspace). The
 * library allocates nothing on the call path, keeps no per-call state, and enqueues its
 * kernels asynchronously on `stream` (a hipStream_t; NULL is the null stream). No call
 * synchronises the host except moe_lora_debug_status. Two calls that share a workspace
 * must be ordered on one stream.
 *
 * Errors: every entry point validates its arguments on the host before enqueueing any work
 * and returns a negative MOELORA_E* code without touching the device when they are invalid.
 * Data-dependent problems (non-finite logits, adapter ids out of range) cannot be seen on the
 * host; kernels record them as flags in the workspace, treat such a token's adapter as -1 and
 * such a logit as -infinity, and moe_lora_debug_status reads the flags back.
 */
#ifndef MOELORA_H
#define MOELORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MOELORA_OK 0
#define MOELORA_EINVAL_DIMS (-1) /* a size is out of the supported range (see below) */
#define MOELORA_ENULL (-2)       /* a required pointer is NULL */
#define MOELORA_EALIGN (-3)      /* a tensor pointer is not 16-byte aligned */
#define MOELORA_EWORKSPACE (-4)  /* workspace too small or misaligned (256-byte alignment) */
#define MOELORA_EHIP (-5)        /* a HIP launch or runtime call failed */
#define MOELORA_EDEVICE (-6)     /* the current device is not gfx950 */
#define MOELORA_EUNSUPPORTED (-7) /* reserved: a combination of arguments this build does not run */
#define MOELORA_ESCRATCH (-8)     /* moe_lora_forward_noalloc: the call needs more than its scratch */

/* Device-side flags reported by moe_lora_debug_status. */
#define MOELORA_FLAG_NONFINITE_LOGIT 1u
#define MOELORA_FLAG_ADAPTER_RANGE 2u

/* Layer sizes (page "vLLM MoE LoRA SageMaker Bedrock", sections "Entendendo os Modelos MoE" and
 * "O Papel da Multi-LoRA": T tokens of width hidden, n_experts experts of intermediate width
 * inter, n_adapters LoRA adapters of rank r). Supported: T >= 0; hidden and inter positive
 * multiples of 128; n_experts in [1, 1024]; n_adapters >= 1; rank in {8, 16, 32, 64};
 * 1 <= topk <= min(n_experts, 16). Buffers the kernels address with 32-bit offsets must stay
 * under 2 GiB: x (T x hidden), the activations (capacity x inter, capacity as reported by
 * moe_lora_workspace_layout, at most T*topk + 255*n_experts rounded up to 256) and one expert's
 * W1 (2*inter x hidden); larger sizes are rejected with MOELORA_EINVAL_DIMS. */
typedef struct {
  int32_t T, hidden, inter, n_experts, n_adapters, rank;
} moe_lora_dims;

/* Dense multi-LoRA (SGMV) sizes: T tokens, in_features (K) and out_features (N) of the
 * projection, n_adapters, rank. Supported: T >= 0; in_features a positive multiple of 128;
 * out_features a positive multiple of 64; n_adapters >= 1; rank in {8, 16, 32, 64}; x (T x K)
 * under 2 GiB. */
typedef struct {
  int32_t T, in_features, out_features, n_adapters, rank;
} moe_lora_sgmv_dims;

/* Bytes of device workspace moe_lora_forward needs for these sizes (0 when the sizes are
 * unsupported): the routing, the pairs sorted by (expert, adapter, token) with their segment
 * table (page "vLLM MoE LoRA SageMaker Bedrock", section "Implementação Técnica no vLLM"; page
 * "Punica: Multi-Tenant LoRA Serving", proposed method), the LoRA shrink outputs z = xA (section
 * "O Papel da Multi-LoRA") and the expert intermediates, sized for the GEMM path these sizes
 * take. The workspace must be 256-byte aligned; its contents need no initialisation and are
 * overwritten by every call. Host-only. */
size_t moe_lora_workspace_size(const moe_lora_dims *d, int32_t topk);

/* The fused layer (page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE":
 * each token goes to its top-k experts, whose gate_up and down outputs are aggregated with the
 * router weights; section "O Papel da Multi-LoRA": every projection with frozen W also adds the
 * token's adapter term xAB, as shrink z = xA then expand zB; section "Implementação Técnica no
 * vLLM": the expert and adapter sparsities handled together). Steps: routing (top-k softmax),
 * sorting token-expert pairs by (expert, adapter, token), LoRA shrink for gate_up, gate_up GEMM
 * with the LoRA expand and SiLU-and-mul fused in its epilogue, LoRA shrink for down, down GEMM
 * with the LoRA expand fused, and the weighted top-k combine. See the header comment for
 * layouts; every pointer is device memory owned by the caller, 16-byte aligned (workspace:
 * 256-byte aligned, at least moe_lora_workspace_size bytes). Returns MOELORA_OK once the work is
 * enqueued on `stream`, or a negative code before any device work (sizes, NULL or misaligned
 * pointers, workspace, device). With T = 0 nothing is enqueued and no pointer is inspected. */
int moe_lora_forward(const void *x, const float *router_logits, const void *W1, const void *W2,
                     const void *A1, const void *B1, const void *A2, const void *B2,
                     const int32_t *adapter_ids, int32_t topk, const moe_lora_dims *d, void *y,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Stages of moe_lora_forward, in launch order: 0 route, 1 align, 2 gate_up LoRA shrink,
 * 3 gate_up GEMM (+ LoRA expand, SiLU-and-mul), 4 down LoRA shrink, 5 down GEMM (+ LoRA
 * expand), 6 combine. */
#define MOELORA_N_STAGES 7

/* moe_lora_forward for measurement (the layer of moe_lora_forward, same passages): additionally records stage_events[i] (caller-created
 * hipEvent_t handles, an array of MOELORA_N_STAGES + 1) on `stream` right before stage i and
 * stage_events[MOELORA_N_STAGES] after the last stage, so the elapsed time between events i
 * and i+1 is stage i. A NULL entry is not recorded (each record adds a gap between launches,
 * so a caller timing one stage passes only its two events). Same results and errors as
 * moe_lora_forward; MOELORA_ENULL when stage_events is NULL. With T = 0 no event is
 * recorded. */
int moe_lora_forward_timed(const void *x, const float *router_logits, const void *W1,
                           const void *W2, const void *A1, const void *B1, const void *A2,
                           const void *B2, const int32_t *adapter_ids, int32_t topk,
                           const moe_lora_dims *d, void *y, void *workspace,
                           size_t workspace_bytes, void *stream, void *const *stage_events);

/* moe_lora_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same layer and results,
 * with the workspace taken from a static device array of 128 MiB inside the library instead of
 * a caller buffer. Each GPU the library runs on holds its own copy of that array from the
 * device's first call until the process ends; the call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine). The caller still passes every input and y, device
 * memory as in moe_lora_forward. Sizes whose workspace (moe_lora_workspace_size) exceeds
 * 128 MiB are rejected with MOELORA_ESCRATCH before any device work: the decode-sized layouts
 * (few token-expert pairs per expert) fit, the tiled layouts of large batches may not. Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents: two calls that overlap on one GPU
 * (different streams, or different threads without ordering) race and must not be issued; calls
 * ordered on one stream are safe. The data flags of moe_lora_debug_status are not readable for
 * these calls. Same other errors as moe_lora_forward. */
int moe_lora_forward_noalloc(const void *x, const float *router_logits, const void *W1,
                             const void *W2, const void *A1, const void *B1, const void *A2,
                             const void *B2, const int32_t *adapter_ids, int32_t topk,
                             const moe_lora_dims *d, void *y, void *stream);

/* Router logits (page "vLLM MoE LoRA SageMaker Bedrock", section "Entendendo os Modelos MoE":
 * the router scores every expert for each token): logits[t][e] = sum_c x[t][c] W_router[e][c],
 * bf16 inputs x [T][hidden] and W_router [n_experts][hidden] (16-byte aligned), fp32 sums,
 * logits [T][n_experts] float32. hidden a positive multiple of 128, n_experts in [1, 1024].
 * Asynchronous on `stream`. */
int moe_lora_router_logits(const void *x, const void *W_router, int32_t T, int32_t hidden,
                           int32_t n_experts, float *logits, void *stream);

/* moe_lora_forward starting from the router weights (page "vLLM MoE LoRA SageMaker Bedrock",
 * section "Entendendo os Modelos MoE": the router scores the experts of each token, then the
 * layer of moe_lora_forward runs): the logits of moe_lora_router_logits go into the workspace
 * (moe_lora_workspace_size covers them) and the layer runs from them, so the result equals
 * moe_lora_forward on those logits. W_router bf16 [n_experts][hidden], 16-byte aligned. Every
 * argument is checked, as in moe_lora_forward, before the router GEMM is enqueued. */
int moe_lora_forward_routed(const void *x, const void *W_router, const void *W1, const void *W2,
                            const void *A1, const void *B1, const void *A2, const void *B2,
                            const int32_t *adapter_ids, int32_t topk, const moe_lora_dims *d,
                            void *y, void *workspace, size_t workspace_bytes, void *stream);

/* moe_lora_forward with FP8 expert weights (page "AWS SageMaker MoE kernel optimizations",
 * third paragraph: FP8 expert weights, their scales applied on the way into the expert
 * GEMMs). W1q [E][2I][h] and W2q [E][h][I] hold OCP E4M3 codes (1 byte each: sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; no infinities) and W1_scale [E][2I], W2_scale [E][h] one
 * float32 per weight row: weight = decode(code) * scale. Everything else (x, the LoRA weights,
 * y, the workspace and its size) is as in moe_lora_forward, device pointers, caller-owned.
 * The codes are 16-byte aligned, the scales 4-byte aligned. Both GEMM regimes take E4M3
 * weights: the weight-streaming one (few token-expert pairs per expert) and the LDS-tiled one
 * (codes staged in LDS as bytes, converted to bf16 after the LDS read); the LoRA weights stay
 * bf16. stage_events, when not NULL, is as in moe_lora_forward_timed. */
int moe_lora_forward_fp8(const void *x, const float *router_logits, const void *W1q,
                         const float *W1_scale, const void *W2q, const float *W2_scale,
                         const void *A1, const void *B1, const void *A2, const void *B2,
                         const int32_t *adapter_ids, int32_t topk, const moe_lora_dims *d,
                         void *y, void *workspace, size_t workspace_bytes, void *stream,
                         void *const *stage_events);

/* Upper bound on the padded sorted-pair length for (seg_pad, block_m) of moe_lora_route_align
 * (pairs grouped by expert and adapter, page "Punica: Multi-Tenant LoRA Serving", proposed
 * method: segments of tokens sharing an adapter): T*topk*seg_pad + n_experts*(block_m-1), or -1
 * for invalid arguments. Host-only. */
int64_t moe_lora_sorted_capacity(const moe_lora_dims *d, int32_t topk, int32_t seg_pad,
                                 int32_t block_m);

/* Bytes of device workspace moe_lora_sgmv needs (0 when the sizes are unsupported): the tokens
 * sorted into adapter segments and the shrink outputs (page "Punica: Multi-Tenant LoRA Serving",
 * proposed method). 256-byte aligned, no initialisation needed. Host-only. */
size_t moe_lora_sgmv_workspace_size(const moe_lora_sgmv_dims *d);

/* Dense multi-LoRA, the per-adapter segmented shrink and expand of one projection (page
 * "Punica: Multi-Tenant LoRA Serving", proposed method: one base model, a batch of tokens
 * with different adapters, the LoRA add applied per segment of tokens sharing an adapter; page
 * "vLLM MoE LoRA SageMaker Bedrock", section "O Papel da Multi-LoRA": z = xA, then zB):
 *   y[t] += (x[t] A[a]^T) B[a]^T,  a = adapter_ids[t]; tokens with a = -1 keep y[t].
 * x [T][K] bf16, A [nA][r][K] bf16, B [nA][N][r] bf16, adapter_ids [T] int32, y [T][N] bf16
 * updated in place (the sum in fp32, rounded once); device pointers, caller-owned, 16-byte
 * aligned. Adapter ids outside [-1, nA) act as -1 and set MOELORA_FLAG_ADAPTER_RANGE
 * (moe_lora_debug_status on this workspace). Asynchronous on `stream`; allocates nothing. */
int moe_lora_sgmv(const void *x, const void *A, const void *B, const int32_t *adapter_ids,
                  const moe_lora_sgmv_dims *d, void *y, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Routing and align on their own, for inspection and tests (page "vLLM MoE LoRA SageMaker
 * Bedrock", section "Entendendo os Modelos MoE": each token's top-k experts and their weights;
 * section "Implementação Técnica no vLLM": the pairs grouped by expert, then by adapter; page
 * "Punica: Multi-Tenant LoRA Serving", proposed method: tokens of one adapter form a segment).
 *   topk_ids   int32 [T][topk]  expert of slot j, slots in descending logit order
 *   topk_w     f32   [T][topk]  softmax of the selected logits
 *   sorted_pairs int32 [sorted_cap]  pair ids p = t*topk + j ordered by the key
 *              (expert, adapter, token); each (expert, adapter) segment padded with -1 to a
 *              multiple of seg_pad, each expert block to a multiple of block_m; entries past
 *              the padded total are left untouched
 *   expert_offsets int32 [E+1]  padded start of each expert block; [E] = padded total
 *   seg_table  int32 [T*topk][4]  rows (expert, adapter, padded start, real count) in key
 *              order (adapter -1 first within an expert)
 *   n_seg      int32 [1]        number of seg_table rows written
 * All outputs are device pointers. seg_pad and block_m are in [1, 256]; sorted_cap must be at
 * least moe_lora_sorted_capacity(...). The workspace is the same as moe_lora_forward's. With
 * T = 0, router_logits, adapter_ids, topk_ids and topk_w may be NULL. */
int moe_lora_route_align(const float *router_logits, const int32_t *adapter_ids, int32_t topk,
                         const moe_lora_dims *d, int32_t seg_pad, int32_t block_m,
                         int32_t *topk_ids, float *topk_w, int32_t *sorted_pairs,
                         int64_t sorted_cap, int32_t *expert_offsets, int32_t *seg_table,
                         int32_t *n_seg, void *workspace, size_t workspace_bytes, void *stream);

/* Where moe_lora_forward (and its _timed, _routed and _fp8 variants) keeps the sorted layout of a
 * call inside the workspace, so that a caller can read the layer's own routing tables back after
 * a call and check them (page "vLLM MoE LoRA SageMaker Bedrock", section "Implementação Técnica
 * no vLLM": token-expert pairs grouped by expert and, inside an expert, by adapter). Offsets are
 * bytes from the start of the workspace; each region holds int32 (topk_w: float32):
 *   topk_ids [T][topk], topk_w [T][topk]     the routing of every token
 *   sorted_pairs [capacity]   pair ids t*topk + j in (expert, adapter, token) order, each expert
 *                             block padded with -1 to a multiple of block_m (seg_pad 1)
 *   expert_offsets [E+1], seg_table [n_seg][4], n_seg [1]   as in moe_lora_route_align
 *   n_blocks [1]              padded total / block_m
 *   block_expert [n_blocks]   expert of each row block
 *   block_seg [n_blocks]      segment holding the block's first row, -1 when that row is padding
 *   pair_row [T*topk]         sorted row of each pair
 *   sorted_ad [capacity]      adapter of each sorted row, -1 for none and for padding rows
 * Only the rows below the padded total are defined. Host-only: touches no device memory.
 * Returns MOELORA_OK, or the error moe_lora_workspace_size would meet (MOELORA_ENULL for a NULL
 * out). */
typedef struct {
  int32_t tiled;    /* 1: LDS-tiled MFMA GEMMs; 0: weight-streaming GEMMs */
  int32_t block_m;  /* row-block size of the sorted layout */
  int64_t capacity; /* rows reserved for sorted_pairs and sorted_ad */
  int64_t workspace_bytes;
  int64_t topk_ids, topk_w, sorted_pairs, expert_offsets, seg_table, n_seg, n_blocks,
      block_expert, block_seg, pair_row, sorted_ad;
} moe_lora_layout_info;

int moe_lora_workspace_layout(const moe_lora_dims *d, int32_t topk, moe_lora_layout_info *out);

/* Text for a return code (the MOELORA_E* codes above; no page defines them). Never NULL; the
 * string is static and owned by the library. */
const char *moe_lora_strerror(int code);

/* Synchronises `stream`, then reads the device flags of the last call that used this
 * workspace into *flags (MOELORA_FLAG_* bits: the data checks that the pages leave open, a
 * non-finite router logit and an adapter id outside [-1, nA), raised by the routing and align
 * kernels of the layer). Returns MOELORA_OK, MOELORA_ENULL, MOELORA_EWORKSPACE (misaligned or
 * under 16 bytes) or MOELORA_EHIP. */
int moe_lora_debug_status(const void *workspace, size_t workspace_bytes, void *stream,
                          uint32_t *flags);

#ifdef __cplusplus
}
#endif

#endif /* MOELORA_H */

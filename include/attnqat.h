/*
 * attnqat.h -- C ABI of the Attn-QAT attention library for AMD Instinct MI355X
 * (gfx950).
 *
 * The library computes quantization-aware-training attention: non-causal
 * softmax attention in which Q, K, V and the probability matrix P are NVFP4
 * fake-quantized (16-element groups, an FP8 E4M3 scale per group, E2M1 values,
 * no global scale), both products take BF16 operands with FP32 accumulation,
 * and the backward pass treats every quantizer as straight-through.
 *
 * Sources (the FastVideo pages this work follows):
 *  - "Attn-QAT Training" guide, section "Architecture-specific Triton
 *    routing": query and key/value lengths may differ (cross-attention), K and
 *    V share a length; the training kernel must fail rather than fall back to
 *    dense attention ("Prerequisites").
 *  - FastVideo VSA checkpoint metadata (vsqa-test-1.3b), keys
 *    attention.precision (quant_p, quant_v, quantize_fine, no global scale
 *    factors, "NVFP4 fake-quant with BF16 matmul"), linear_quantization.format
 *    (the NVFP4 block format), attention.selection and cube_shape (block
 *    sparse selection over 128-token blocks).
 *  - fastvideo-kernel commit message, SM100 Attn-QAT route paragraph: the
 *    forward saves softmax statistics, the backward recomputes P, and outputs,
 *    statistics and gradients are bitwise reproducible.
 *  - Attn-QAT inference backend pull request, review finding on sm_scale: the
 *    softmax scale passed by the caller must be honoured; the review's note on
 *    in-place K smoothing: inputs must not be modified.
 *
 * Conventions shared by every entry point
 *  - Tensors are bfloat16 (raw 16-bit patterns) in a [B, H, N, D] index space
 *    with the last dimension contiguous. Element strides for the B, H and N
 *    axes are given per tensor (attnqat_strides); an all-zero triple means the
 *    contiguous layout {H*N*D, N*D, D}. Pointers must be 16-byte aligned and
 *    every stride a multiple of 8 elements.
 *  - All pointers to tensor data, statistics and workspaces are device
 *    pointers. The caller owns every buffer; the library allocates no device
 *    memory and keeps no state besides a per-device architecture check and
 *    the optional per-thread kernel-timing record (attnqat_profile_enable).
 *  - All work is enqueued in order on `stream` (a hipStream_t; NULL is the
 *    default stream). No call synchronises the host; results are valid once
 *    the caller has synchronised the stream.
 *  - Inputs are never written.
 *  - Results are bitwise reproducible run to run (no atomics, fixed
 *    accumulation order).
 *  - Arguments are validated before any HIP call. On failure a call returns a
 *    non-zero status, enqueues nothing, and attnqat_last_error() describes the
 *    problem. There is no fallback path.
 */
#ifndef ATTNQAT_H
#define ATTNQAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTNQAT_ABI_VERSION 5

/* status codes */
#define ATTNQAT_OK 0
#define ATTNQAT_E_INVALID 1     /* null pointer, bad size, bad mask, bad scale, aliasing */
#define ATTNQAT_E_UNSUPPORTED 2 /* head dim not 64/128, B*H > 65535, Nq or Nk above
                                 * ATTNQAT_MAX_TOKENS, device is not gfx950 */
#define ATTNQAT_E_MISALIGNED 3  /* pointer not 16-byte aligned or stride not a multiple of 8 */
#define ATTNQAT_E_WORKSPACE 4   /* workspace missing or too small */
#define ATTNQAT_E_HIP 5         /* a HIP call or kernel launch failed */

/* longest query or key sequence the attention entry points accept */
#define ATTNQAT_MAX_TOKENS 4194304

/* quantization mask bits: which operands are NVFP4 fake-quantized */
#define ATTNQAT_QUANT_Q 1u
#define ATTNQAT_QUANT_K 2u
#define ATTNQAT_QUANT_V 4u
#define ATTNQAT_QUANT_P 8u
#define ATTNQAT_QUANT_ALL 15u

/* which probabilities the P quantizer sees (attnqat_problem.p_mode) */
#define ATTNQAT_P_NORMALISED 0u /* P = exp(S - LSE), quantized per 16-key group (default) */
#define ATTNQAT_P_ROWMAX 1u     /* exp(S - m), m = row maximum, quantized, then divided by l */

/* group axis of the standalone fake quantizer */
#define ATTNQAT_AXIS_D 0 /* 16 consecutive elements of the last (head) dimension: Q, K */
#define ATTNQAT_AXIS_N 1 /* 16 consecutive tokens of one column: V */

typedef struct {
    int64_t b, h, n; /* element strides of the B, H and N axes; {0,0,0} = contiguous */
} attnqat_strides;

typedef struct {
    int64_t B, H;   /* batch and heads, >= 1 */
    int64_t Nq, Nk; /* query tokens and key/value tokens, >= 1 */
    int64_t D;      /* head dimension: 64 or 128 */
    float sm_scale; /* softmax scale, used verbatim; finite and > 0 */
    uint32_t quant_mask; /* OR of ATTNQAT_QUANT_* bits (0 = plain attention) */
    attnqat_strides q, k, v, o, dout, dq, dk, dv;
    /* Block-sparse fine attention (VSA-style), NULL for dense attention.
     * Device array int32 [B, H, ceil(Nq/block_tokens), topk] (contiguous) of
     * key-block indices, strictly ascending within each row, each in
     * [0, ceil(Nk/block_tokens)). Query block i attends only to the keys of
     * the listed key blocks; LSE and P are taken over those keys only.
     * attnqat_fwd and attnqat_bwd check these rules on the device before any
     * sparse kernel reads the index: if an entry breaks them, the attention
     * kernels do no work, every output of the call is filled with NaN, and
     * attnqat_block_idx_status reports the failure. */
    const int32_t* kv_block_idx;
    int32_t topk;         /* entries per row of kv_block_idx (ignored when dense) */
    int32_t block_tokens; /* tokens per block; must be 128 when kv_block_idx != NULL;
                           * block-sparse problems have at most 1024 blocks per sequence */
    /* Row-max-relative P quantization (an alternative reading of which P the
     * pages quantize: the inference-backend pull request's FP4 attention call
     * takes a single_level_p_quant option). With p_mode == ATTNQAT_P_ROWMAX
     * and the P bit set, the quantized quantity is exp(S - m), m_i = max_j
     * S_ij (over the keys the row attends to), and O = FQ(exp(S - m)) V / l
     * with l_i = exp(LSE_i - m_i); the backward uses the same Pq. Zero
     * (ATTNQAT_P_NORMALISED) keeps the normalised P. */
    uint32_t p_mode;
    /* Row maxima m of S, device fp32 [B,H,Nq] contiguous, 4-byte aligned:
     * written by attnqat_fwd and read by attnqat_bwd when p_mode is
     * ATTNQAT_P_ROWMAX (required then, and must not overlap any other
     * argument); ignored otherwise. */
    float* row_max;
    /* Optional second forward output (NULL: not formed), bf16 [B,H,Nq,D] with
     * the strides of o: O_ste = P FQ_tokens(V) with the unquantized P (the
     * P of p_mode), the straight-through counterpart of O. Passing it as the
     * backward's `o` gives the additive straight-through delta
     * Dl = rowsum(dout * O_ste) (the pages' SM120 route joins a quantized and
     * an STE P@V). */
    void* o_ste;
} attnqat_problem;

/* ABI version of the loaded library (ATTNQAT_ABI_VERSION it was built with). */
int attnqat_abi_version(void);

/* Static description of a status code. */
const char* attnqat_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
const char* attnqat_last_error(void);

/*
 * NVFP4 fake quantization, y = FQ(x) (VSA checkpoint metadata,
 * linear_quantization.format, with no global scale as in attention.precision).
 * For each group of 16 consecutive elements along `group_axis` (groups start at
 * index 0; a partial last group is padded with zeros):
 *   s = E4M3(max|x| / 6)   round to nearest even, saturating at 448
 *   y = sign(x) * E2M1(|x| / s) * s   round to nearest even on
 *       {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6; s == 0 gives signed 0.
 * The result is exact: y is bitwise identical to an exact-arithmetic
 * evaluation of these steps.
 *   x, y        bf16 tensors [B,H,N,D] with strides xs, ys (y may not overlap x)
 *   scale_codes optional (NULL allowed) uint8 OCP E4M3FN codes, contiguous
 *               [B,H,N,D/16] for ATTNQAT_AXIS_D, [B,H,ceil(N/16),D] for
 *               ATTNQAT_AXIS_N.
 *   D           a multiple of 16 (axis D) or of 8 (axis N), at most 1024.
 */
int attnqat_fakequant_nvfp4(const void* x, attnqat_strides xs, void* y, attnqat_strides ys,
                            uint8_t* scale_codes, int64_t B, int64_t H, int64_t N, int64_t D,
                            int group_axis, void* stream);

/*
 * Workspace bytes attnqat_fwd needs for problem p: the quantized operand
 * copies and, for a dense problem with the P quantizer whose pass 2 leaves
 * its last round of workgroups (one per compute unit, planned for 256) at
 * most 4/5 full, the fp32 partial sums of that round (at most 64 MiB at
 * D = 128). Depends on p only.
 */
size_t attnqat_fwd_workspace_bytes(const attnqat_problem* p);

/*
 * Forward pass of quantization-aware attention. Definition: the VSA
 * checkpoint metadata, attention.precision ("NVFP4 fake-quant with BF16
 * matmul", quant_p and quant_v set, no global scale factors), for which
 * operands are quantized and in which number format the products run; the
 * Attn-QAT training guide (FWD_EXACT_M row of its environment table) and the
 * fastvideo-kernel commit message (SM100 route paragraph) for the softmax
 * statistics the forward saves and the backward reuses, which make the
 * quantized P that of the normalised probabilities. Writes
 *   o    bf16 [B,H,Nq,D] (strides p->o):  O = FQ_keys(P) FQ_tokens(V)
 *   lse  fp32 [B,H,Nq] contiguous:        LSE = ln sum_j exp(S_ij)
 * with S = sm_scale FQ_d(Q) FQ_d(K)^T and P = exp(S - LSE) (normalised); each
 * quantizer applies only if its mask bit is set. P is quantized per 16-key
 * group of each query row, groups aligned at key 0; there is no
 * renormalisation after quantization. With p_mode == ATTNQAT_P_ROWMAX (and
 * the P bit set) O = FQ_keys(exp(S - m)) FQ_tokens(V) / l instead, and the row
 * maxima m are also written to p->row_max.
 * `workspace` (device, 256-byte aligned) of at least
 * attnqat_fwd_workspace_bytes(p) bytes is scratch owned by the caller; its
 * contents are undefined afterwards.
 */
int attnqat_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v, void* o,
                float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attnqat_fwd without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments, results and errors as attnqat_fwd
 * (the caller still passes every input and output); the scratch is a fixed
 * 64 MiB device buffer inside the library, one per GPU, held until the
 * process ends. The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Problems whose attnqat_fwd_workspace_bytes
 * exceed 67108864 are rejected with ATTNQAT_E_UNSUPPORTED. Every call on a
 * GPU shares that GPU's buffer, which keeps the last call's contents (the
 * forward writes every scratch byte it reads, so nothing needs clearing):
 * calls that overlap on one GPU, from several streams or threads, race.
 */
int attnqat_fwd_noalloc(const attnqat_problem* p, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* stream);

/* Workspace bytes attnqat_bwd needs for problem p. */
size_t attnqat_bwd_workspace_bytes(const attnqat_problem* p);

/*
 * Backward pass with straight-through quantizers. Definition: the Attn-QAT
 * training guide and the fastvideo-kernel commit message (SM100 route
 * paragraph: the backward recomputes P from the saved statistics, with
 * bitwise reproducible gradients) and the VSA checkpoint metadata's
 * attention.precision (the same quantizers as the forward). Given the forward inputs,
 * the forward output `o` and statistics `lse` (as written by attnqat_fwd) and
 * the output gradient `dout`, writes bf16 dq, dk, dv:
 *   Dl = rowsum(dout * o)
 *   dP = dout FQ_tokens(V)^T,  dS = P * (dP - Dl)   (P unquantized, from lse)
 *   dV = FQ_keys(P)^T dout    (FQ_keys(exp(S - m))^T dout / l with ATTNQAT_P_ROWMAX,
 *                              m read from p->row_max as written by attnqat_fwd)
 *   dQ = sm_scale dS FQ_d(K),  dK = sm_scale dS^T FQ_d(Q)
 * Outputs must not overlap each other or any input.
 */
int attnqat_bwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Result of the device-side check of p->kv_block_idx made by the last
 * block-sparse attnqat_fwd or attnqat_bwd that used `workspace` (the same
 * pointer, with that call's work enqueued on `stream` or completed). Enqueues
 * a 4-byte copy on `stream`, waits for it, and sets *invalid to 1 if the index
 * broke its rules (the call's outputs are then NaN), else 0. Undefined after a
 * dense call, which does not run the check.
 */
int attnqat_block_idx_status(const void* workspace, int* invalid, void* stream);

/*
 * Key blocks kept per query block by the pages' selection rule (VSA
 * checkpoint metadata, attention.selection: effective_topk =
 * max(1, min(ceil((1 - sparsity) num_blocks), num_blocks)), evaluated in
 * double precision). Returns the count, or -ATTNQAT_E_INVALID if num_blocks
 * < 1 or sparsity is outside [0, 1]. Host-only; enqueues nothing.
 */
int attnqat_effective_topk(int64_t num_blocks, double sparsity);

/* Workspace bytes attnqat_block_select needs. */
size_t attnqat_block_select_workspace_bytes(const attnqat_problem* p);

/*
 * VSA-style coarse block selection (checkpoint metadata, attention.selection
 * and precision.coarse = BF16, quantize_coarse = false). Q and K are
 * mean-pooled over blocks of p->block_tokens tokens (a partial last block over
 * its own tokens); the means and the block scores qbar_i . kbar_j are rounded
 * to bfloat16 from their exact values; each query block keeps the p->topk
 * highest-scoring key blocks (ties to the lower index), written ascending to
 * kv_block_idx, int32 [B, H, ceil(Nq/bt), topk]. p->kv_block_idx is ignored.
 * topk must be in [1, ceil(Nk/bt)] and ceil(Nk/bt) <= 1024.
 */
int attnqat_block_select(const attnqat_problem* p, const void* q, const void* k,
                         int32_t* kv_block_idx, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Workspace bytes attnqat_vsa_fwd and attnqat_vsa_bwd need (one size for both). */
size_t attnqat_vsa_workspace_bytes(const attnqat_problem* p);

/*
 * VSA coarse branch and its gated combination with the fine branch
 * (checkpoint metadata: attention kind vsa, backend VSA_QAT_TRAIN_C128,
 * precision.coarse = BF16 with quantize_coarse = false, compression_gates
 * trained; the fastvideo-kernel commit message scatters the gate with Q, K and
 * V, so the gate is a per-token [B,H,Nq,D] tensor). With blocks of
 * p->block_tokens (must be 128) tokens, a partial last block averaged over its
 * own tokens, and Qbar, Kbar, Vbar the bf16-rounded block means of the raw q,
 * k, v (as for attnqat_block_select):
 *   O_c = softmax(sm_scale Qbar Kbar^T) Vbar   (fp32 from the bf16 means)
 *   o   = o_fine + gate * O_c[block(t)]        (bf16, rounded once)
 * o_fine is the fine branch's output (attnqat_fwd with kv_block_idx). gate,
 * o_fine and o are bf16 [B,H,Nq,D] with the strides of p->o; q, k, v use their
 * own. o must not overlap any input or the workspace. ceil(Nq/128) and
 * ceil(Nk/128) must be at most 1024. p->quant_mask, p_mode and kv_block_idx
 * are not used (the coarse branch is never quantized).
 */
int attnqat_vsa_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                    const void* gate, const void* o_fine, void* o, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Backward of the coarse branch and the combination, to be run after
 * attnqat_bwd of the fine branch (called with o = o_fine, so that its softmax
 * delta is rowsum(dout * o_fine)). Adds in place to dq, dk, dv (bf16, which
 * hold the fine gradients) the coarse contributions: dO_c[i] = sum over the
 * tokens of query block i of gate * dout, dS = P (dO_c Vbar^T - rowsum(dO_c
 * O_c)), dQbar = sm_scale dS Kbar, dKbar = sm_scale dS^T Qbar, dVbar = P^T
 * dO_c, and every token of a block receives its block mean's gradient divided
 * by the block's token count. Writes dgate = dout * O_c[block(t)] (bf16, the
 * strides of p->o) unless dgate is NULL. dq, dk, dv and dgate must not overlap
 * each other, any input or the workspace.
 */
int attnqat_vsa_bwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                    const void* gate, const void* dout, void* dq, void* dk, void* dv,
                    void* dgate, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attnqat_mxfp4_fwd needs for problem p (0 if p is invalid). */
size_t attnqat_mxfp4_fwd_workspace_bytes(const attnqat_problem* p);

/*
 * Real-FP4 inference attention forward on MXFP4 operands: this chip's
 * counterpart of the pages' real-FP4 inference attention (the inference
 * backend pull request's FP4 attention call with single-level P
 * quantization; the Attn-QAT guide's inference route), computed with the
 * scaled FP4 matrix instruction. Its block format is MX, not NVFP4: every 32
 * consecutive values share one power-of-two (E8M0) scale
 *   X = 2^(floor(log2 amax) - 2)   (a block of zeros: 2^-127)
 *   MX(x) = X E2M1(x / X)          round to nearest even, saturating at 6,
 * with blocks along d for Q and K, along the tokens for V and along the keys
 * for P, each starting at index 0 (a partial last block padded with zeros).
 * Writes
 *   o    bf16 [B,H,Nq,D] (strides p->o):  O = MX(P~) MX(V) / l
 *   lse  fp32 [B,H,Nq] contiguous:        LSE = m + ln l
 * with S = sm_scale MX(Q) MX(K)^T, m_i = max_j S_ij, P~ = exp(S - m) and
 * l_i = sum_j P~_ij (unquantized). Requirements: quant_mask ==
 * ATTNQAT_QUANT_ALL, kv_block_idx == NULL and o_ste == NULL (else
 * ATTNQAT_E_UNSUPPORTED); p_mode and row_max are not used. Other arguments,
 * alignment, overlap and error rules are those of attnqat_fwd; `workspace`
 * (device, 256-byte aligned, attnqat_mxfp4_fwd_workspace_bytes(p) bytes) is
 * scratch owned by the caller and holds the quantized operands afterwards.
 */
int attnqat_mxfp4_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                      void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing (diagnostics). While enabled on the calling thread, every
 * kernel the library enqueues from that thread is bracketed by a pair of HIP
 * events recorded on the kernel's own stream (so only the kernel's execution is
 * timed). attnqat_profile_read synchronises on the recorded events, writes for
 * up to max_kinds kernel kinds their name (static string), total milliseconds
 * and launch count, clears the record, and returns the number of kinds
 * written (negative status on a HIP failure). Enabling or disabling clears the
 * record. Event pairs are created on first use and reused; at most 65536
 * launches are recorded between reads (later ones are not timed).
 */
int attnqat_profile_enable(int on);
int attnqat_profile_read(const char** names, double* total_ms, int* launches, int max_kinds);

#ifdef __cplusplus
}
#endif

#endif /* ATTNQAT_H */

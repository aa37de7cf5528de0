// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include "aq_common.h"

namespace aq {

// Tile sizes shared by the host planner and the kernels.
constexpr int kTileN = 256;  // token padding granularity of every workspace operand

// Dense dK/dV: most parts a key block is split into, and most split blocks
// (fewer than one round of workgroups on a chip of 256 compute units).
constexpr int kMaxDkdvParts = 4;
constexpr int kMaxDkdvSplit = 255;
// Compute units the workspace planner assumes when it sizes the dQ and
// forward pass-2 partial regions (MI355X); a device with another count
// splits only when its own split fits the region.
constexpr int kPlanCus = 256;
// Fewest key tiles a last-round workgroup of a split dQ or pass-2 launch
// takes.
constexpr int kMinChunkTiles = 8;

// Size of the fixed device scratch behind attnqat_fwd_noalloc (aq_noalloc.hip)
// and the lookup of its address on the current device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(int dev, void** out);

struct FqArgs {
    const uint16_t* x;
    int64_t xsb, xsh, xsn;
    uint16_t* y;
    int64_t ysb, ysh, ysn;
    uint8_t* codes;  // nullable
    int64_t BH;
    int64_t H;
    int64_t N;     // valid tokens
    int64_t Nout;  // rows written (>= N; rows >= N are zero)
    int D;
};

struct PreArgs {
    const uint16_t* o;
    int64_t osb, osh, osn;
    const uint16_t* dout;
    int64_t dsb, dsh, dsn;
    const float* lse;  // [BH][Nq]
    float* delta;      // [BH][Nq_pad]
    float* lse2;       // [BH][Nq_pad]
    uint16_t* dOw;     // [BH][Nq_pad][D]
    // row-max-relative P quantization (NULL row_max: off): the dK/dV kernel
    // gets dO and Dl scaled per row by 1/l = exp2(m2 - lse2) and m2 = m log2(e)
    // in place of lse2, so that it quantizes exp(S - m) and its products
    // carry the 1/l
    const float* row_max;  // [BH][Nq]
    float* delta_kv;       // [BH][Nq_pad]
    float* lse2_kv;        // [BH][Nq_pad]
    uint16_t* dOw_kv;      // [BH][Nq_pad][D]
    int64_t BH, H, Nq, Nq_pad;
    int D;
};

// Attention problem as seen by the tiled kernels: operands live in the
// workspace, contiguous and zero-padded to multiples of kTileN tokens.
struct AttnArgs {
    const uint16_t* Qw;   // [BH][Nq_pad][D]
    const uint16_t* Kw;   // [BH][Nk_pad][D]
    const uint16_t* Vw;   // [BH][Nk_pad][D]
    const uint16_t* Kt;   // [BH][D][Nk_pad] permuted
    const uint16_t* Vt;   // [BH][D][Nk_pad] natural token order; fp16 when pv_f16
    const uint16_t* dOw;  // [BH][Nq_pad][D]
    const float* lse;     // forward: natural-log LSE output/input [BH][Nq]
    const float* lse2;    // backward: LSE * log2(e), [BH][Nq_pad]
    const float* delta;   // backward: [BH][Nq_pad]
    float* lse_out;       // forward pass 1 output [BH][Nq]
    float* row_max_out;   // forward pass 1: row maxima of S [BH][Nq] (NULL: not written)
    const float* row_max; // forward pass 2: quantize exp(S - m) and scale O by 1/l (NULL: off)
    uint16_t* o;          // strided outputs
    uint16_t* o_ste;      // forward: P Vq with the unquantized P (o's strides; NULL: not formed)
    int64_t osb, osh, osn;
    uint16_t* dq;
    int64_t dqsb, dqsh, dqsn;
    uint16_t* dk;
    int64_t dksb, dksh, dksn;
    uint16_t* dv;
    int64_t dvsb, dvsh, dvsn;
    // block sparsity (NULL = dense)
    const int32_t* kv_idx;   // [BH][nbq][topk]
    const int32_t* q_list;   // [BH][nbk][nbq] reverse index (query blocks per key block)
    const int32_t* q_count;  // [BH][nbk]
    const int32_t* kv_order; // [BH][nbk] key blocks of each head by descending count
    const int32_t* idx_err;  // block-index check flag: the sparse kernels skip their work if set
    // dense dK/dV: key blocks [0, dkdv_full) run whole, the others are split
    // into dkdv_parts parts along the queries whose fp32 partial sums
    // [split block][part][dK, dV][128 keys][D] the fixup adds
    float* dkdv_part;
    int dkdv_full, dkdv_parts;
    // dense dQ and dense forward pass 2 (P quantized, no O_ste): query blocks
    // (256 queries, head-major) [0, *_full) run whole, one workgroup each;
    // with *_chunk > 0 the remaining blocks' key tiles are shared out to
    // *_chunks further workgroups, *_chunk consecutive tiles each, whose
    // fp32 partial sums ([slot][256 queries][D], two slots per workgroup) a
    // fixup adds. dQ uses the dK/dV partial region (free once its fixup has
    // run).
    float* dq_part;
    int dq_full, dq_chunk, dq_chunks;
    float* fo_part;
    int fo_full, fo_chunk, fo_chunks;
    int topk;
    int nbq, nbk;
    int64_t H;
    int Nq, Nk, Nq_pad, Nk_pad;
    int BH;
    float c;        // sm_scale * log2(e)
    float sm_scale;
    int quant_p;
    int pv_f16;  // forward: P and V both quantized, P V runs on fp16 operands
};

hipError_t launch_fq_axis_d(const FqArgs& a, bool quant, hipStream_t st);
hipError_t launch_fq_axis_n(const FqArgs& a, bool quant, hipStream_t st);
// FQ along the tokens (quant) written transposed to y = [BH][D][Nout]
// (contiguous; fp16 with to_f16). Nout and D multiples of 64.
hipError_t launch_fq_n_transpose(const FqArgs& a, bool quant, bool to_f16, hipStream_t st);
hipError_t launch_transpose_perm(const uint16_t* src, uint16_t* dst, int64_t BH, int Npad, int D,
                                 bool perm, bool to_f16, hipStream_t st);
hipError_t launch_bwd_pre(const PreArgs& a, hipStream_t st);

hipError_t launch_fwd_lse(const AttnArgs& a, int D, hipStream_t st);
hipError_t launch_fwd_out(const AttnArgs& a, int D, hipStream_t st);
// forward without P quantization: O, LSE (and row maxima) in one pass
hipError_t launch_fwd_single(const AttnArgs& a, int D, hipStream_t st);
hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t st);
hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t st);

struct SelectArgs {
    const uint16_t* q;
    int64_t qsb, qsh, qsn;
    const uint16_t* k;
    int64_t ksb, ksh, ksn;
    uint16_t* qbar;   // [BH][nbq][D] bf16
    uint16_t* kbar;   // [BH][nbk][D] bf16
    int32_t* idx;     // [BH][nbq][topk]
    int32_t* q_list;  // nullable: reverse index [BH][nbk][nbq]
    int32_t* q_count; // nullable: [BH][nbk]
    int64_t BH, H;
    int Nq, Nk, bt, nbq, nbk, topk, D;
};
// VSA coarse branch and gated combination (aq_vsa.hip). Token tensors are
// strided bf16 [B,H,N,D]; gate, o_fine, o and dgate share o's strides.
// Workspace arrays are contiguous per (bh, block).
constexpr int kVsaMaxBlocks = 1024;
struct VsaArgs {
    const uint16_t* q;
    int64_t qsb, qsh, qsn;
    const uint16_t* k;
    int64_t ksb, ksh, ksn;
    const uint16_t* v;
    int64_t vsb, vsh, vsn;
    const uint16_t* gate;
    const uint16_t* o_fine;
    uint16_t* o;
    uint16_t* dgate;  // nullable
    int64_t osb, osh, osn;
    const uint16_t* dout;
    int64_t dsb, dsh, dsn;
    uint16_t* dq;
    int64_t dqsb, dqsh, dqsn;
    uint16_t* dk;
    int64_t dksb, dksh, dksn;
    uint16_t* dv;
    int64_t dvsb, dvsh, dvsn;
    uint16_t *qbar, *kbar, *vbar;  // [BH][nb][D] bf16 block means
    float* oc;                     // [BH][nbq][D] coarse output
    float* lsec;                   // [BH][nbq] coarse LSE
    float* doc;                    // [BH][nbq][D] gradient of the coarse output
    float* dcc;                    // [BH][nbq] rowsum(dO_c O_c)
    float *dqb, *dkb, *dvb;        // [BH][nb][D] gradients of the block means
    int64_t BH, H;
    int Nq, Nk, bt, nbq, nbk, D;
    float sm_scale;
};
hipError_t launch_vsa_pool(const VsaArgs& a, hipStream_t st);
hipError_t launch_vsa_coarse_fwd(const VsaArgs& a, hipStream_t st);
hipError_t launch_vsa_combine(const VsaArgs& a, hipStream_t st);
hipError_t launch_vsa_gate_reduce(const VsaArgs& a, hipStream_t st);
hipError_t launch_vsa_coarse_bwd(const VsaArgs& a, hipStream_t st);
hipError_t launch_vsa_grad_add(const VsaArgs& a, hipStream_t st);

// Real-FP4 (MXFP4) inference forward. Workspace operands: Q and K rows as
// packed E2M1 codes [BH][N_pad][D / 2] bytes with E8M0 scales [BH][N_pad][D / 32];
// V^T codes [BH][D][Nk_pad / 2] with scales [BH][Nk_pad / 64][D][2] (tile by tile).
struct MxArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn;
    uint8_t *qm, *qs, *km, *ks, *vtm, *vts;
    uint16_t* o;
    int64_t osb, osh, osn;
    float* lse;  // [BH][Nq]
    int64_t BH, H;
    int Nq, Nk, Nq_pad, Nk_pad, D;
    float c;  // sm_scale * log2(e)
};
hipError_t launch_mx_quant(const MxArgs& a, hipStream_t st);
hipError_t launch_mx_fwd(const MxArgs& a, hipStream_t st);

hipError_t launch_block_pool(const SelectArgs& a, hipStream_t st);
hipError_t launch_block_topk(const SelectArgs& a, hipStream_t st);
hipError_t launch_reverse_index(const int32_t* idx, int32_t* q_list, int32_t* q_count, int64_t BH,
                                int nbq, int nbk, int topk, int32_t* kv_order,
                                const int32_t* idx_err, hipStream_t st);

// Block-index check (flag = 1 when an entry is out of range or a row is not
// strictly ascending) and the NaN fill of a call's outputs when it is set.
struct PoisonArgs {
    const int32_t* flag;
    uint16_t* t[4];  // strided bf16 [B,H,N[i],D] token tensors
    int64_t sb[4], sh[4], sn[4], N[4];
    int nt;
    float* f[2];  // contiguous fp32 arrays of fn[i] elements
    int64_t fn[2];
    int nf;
    int64_t BH, H;
    int D;
};
hipError_t launch_check_index(const int32_t* idx, int64_t rows, int topk, int nbk, int32_t* flag,
                              hipStream_t st);
hipError_t launch_poison_outputs(const PoisonArgs& a, hipStream_t st);

}  // namespace aq

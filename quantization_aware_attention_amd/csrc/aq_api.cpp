// C ABI of the Attn-QAT library: argument validation, workspace planning and
// kernel launch order. See include/attnqat.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attnqat.h"
#include "aq_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return ATTNQAT_OK;
}

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
int g_dev_arch[kMaxDevices];
std::mutex g_dev_mu;

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTNQAT_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTNQAT_E_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_arch[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(ATTNQAT_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        g_dev_arch[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        if (g_dev_arch[dev] == 2)
            return fail(ATTNQAT_E_UNSUPPORTED, "device %d is %s, this library is built for gfx950",
                        dev, prop.gcnArchName);
    }
    if (g_dev_arch[dev] != 1)
        return fail(ATTNQAT_E_UNSUPPORTED, "device %d is not gfx950", dev);
    return ATTNQAT_OK;
}

// Compute units of the current device (cached per device; 256 on gfx950).
int g_dev_cus[kMaxDevices];
int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        g_dev_cus[dev] = n;
    }
    return g_dev_cus[dev];
}

// Parts to split each of the F workgroups of a launch's last, partial round
// into (rounds of one workgroup per compute unit): the P <= kMaxDkdvParts,
// at most `units` (a part has at least one tile), that minimises the last
// round's length ceil(F P / CUs) / P; 1 when the last round is full.
int split_parts(int64_t F, int cus, int64_t units) {
    int P = 1;
    if (F == 0) return 1;
    for (int c = 2; c <= aq::kMaxDkdvParts && c <= units; ++c)
        if ((double)((F * c + cus - 1) / cus) / c < (double)((F * P + cus - 1) / cus) / P) P = c;
    return P;
}

// Last-round split of a launch over nblk blocks of nt key tiles, one
// workgroup per block per compute unit (dense dQ and forward pass 2): full
// workgroups, and the tiles per further workgroup (chunk, 0: no split) and
// their count (chunks) that spread the F = nblk % cus blocks of the last
// round over up to `cus` workgroups of at least kMinChunkTiles tiles each.
// A last round more than 4/5 full is left whole: the chip runs a partly
// idle round at a higher clock, and at 86% (220 of 256 blocks, 6 heads x
// 31,200 tokens) spreading it measured 1-3% slower with the fixup, against
// 3-8% faster at 59% and 9% full.
struct StreamSplit {
    int64_t full, chunk, chunks;
};
StreamSplit stream_split(int64_t nblk, int64_t nt, int cus) {
    const int64_t F = nblk % cus, total = F * nt;
    int64_t g = total / aq::kMinChunkTiles;
    if (g > cus) g = cus;
    if (F == 0 || g <= F || 5 * F > 4 * (int64_t)cus) return {nblk, 0, 0};  // nothing to gain
    const int64_t chunk = (total + g - 1) / g;
    return {nblk - F, chunk, (total + chunk - 1) / chunk};
}

int hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(ATTNQAT_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return ATTNQAT_OK;
}

// ---------------------------------------------------------------------------
// optional per-thread kernel timing
enum Kind {
    K_FQ_D, K_FQ_N, K_TRANSPOSE, K_FWD_LSE, K_FWD_OUT, K_FWD_SINGLE, K_BWD_PRE, K_BWD_DKDV, K_BWD_DQ,
    K_BLOCK_POOL, K_BLOCK_TOPK, K_REVERSE_INDEX, K_VSA_POOL, K_VSA_COARSE, K_VSA_COMBINE,
    K_VSA_GATE, K_VSA_COARSE_BWD, K_VSA_GRAD_ADD, K_MX_QUANT, K_MX_FWD, K_CHECK_INDEX, K_POISON,
    K_NUM
};
const char* const kKindName[K_NUM] = {
    "fq_axis_d", "fq_axis_n", "transpose_perm", "fwd_lse", "fwd_out", "fwd_single", "bwd_pre", "bwd_dkdv",
    "bwd_dq", "block_pool", "block_topk", "reverse_index", "vsa_pool", "vsa_coarse",
    "vsa_combine", "vsa_gate_reduce", "vsa_coarse_bwd", "vsa_grad_add", "mx_quant", "mx_fwd",
    "check_index", "poison_outputs"};

constexpr int kMaxTimed = 65536;

struct Profiler {
    bool on = false;
    std::vector<hipEvent_t> ev;  // pairs
    std::vector<int> kind;       // kind of recorded pair i
    int used = 0;
};
thread_local Profiler g_prof;

int launch(Kind k, hipStream_t st, hipError_t (*fn)(const void*, hipStream_t), const void* args,
           const char* what) {
    Profiler& P = g_prof;
    const bool timed = P.on && P.used < kMaxTimed;
    if (timed) {
        if ((int)P.kind.size() <= P.used) {
            hipEvent_t a, b;
            if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess)
                return fail(ATTNQAT_E_HIP, "hipEventCreate failed");
            P.ev.push_back(a);
            P.ev.push_back(b);
            P.kind.push_back(0);
        }
        P.kind[P.used] = k;
        int rc = hip_check(hipEventRecord(P.ev[2 * P.used], st), "hipEventRecord");
        if (rc) return rc;
    }
    int rc = hip_check(fn(args, st), what);
    if (rc) return rc;
    if (timed) {
        rc = hip_check(hipEventRecord(P.ev[2 * P.used + 1], st), "hipEventRecord");
        if (rc) return rc;
        ++P.used;
    }
    return ATTNQAT_OK;
}

template <class A, hipError_t (*F)(const A&, hipStream_t)>
hipError_t thunk(const void* a, hipStream_t st) {
    return F(*(const A*)a, st);
}

struct TransposeArgs {
    const uint16_t* src;
    uint16_t* dst;
    int64_t BH;
    int Npad, D;
    bool perm, to_f16;
};
hipError_t do_transpose(const TransposeArgs& t, hipStream_t st) {
    return aq::launch_transpose_perm(t.src, t.dst, t.BH, t.Npad, t.D, t.perm, t.to_f16, st);
}
struct DimArgs {
    aq::AttnArgs a;
    int D;
};
hipError_t do_fwd_lse(const DimArgs& d, hipStream_t st) { return aq::launch_fwd_lse(d.a, d.D, st); }
hipError_t do_fwd_out(const DimArgs& d, hipStream_t st) { return aq::launch_fwd_out(d.a, d.D, st); }
hipError_t do_fwd_single(const DimArgs& d, hipStream_t st) {
    return aq::launch_fwd_single(d.a, d.D, st);
}
hipError_t do_bwd_dq(const DimArgs& d, hipStream_t st) { return aq::launch_bwd_dq(d.a, d.D, st); }
hipError_t do_bwd_dkdv(const DimArgs& d, hipStream_t st) {
    return aq::launch_bwd_dkdv(d.a, d.D, st);
}
hipError_t do_fq_d_q(const aq::FqArgs& a, hipStream_t st) { return aq::launch_fq_axis_d(a, true, st); }
hipError_t do_fq_d_c(const aq::FqArgs& a, hipStream_t st) { return aq::launch_fq_axis_d(a, false, st); }
hipError_t do_fq_n_q(const aq::FqArgs& a, hipStream_t st) { return aq::launch_fq_axis_n(a, true, st); }
hipError_t do_fq_n_c(const aq::FqArgs& a, hipStream_t st) { return aq::launch_fq_axis_n(a, false, st); }
struct FqtArgs {
    aq::FqArgs a;
    bool quant, to_f16;
};
hipError_t do_fq_nt(const FqtArgs& t, hipStream_t st) {
    return aq::launch_fq_n_transpose(t.a, t.quant, t.to_f16, st);
}
struct RevArgs {
    const int32_t* idx;
    int32_t *q_list, *q_count;
    int64_t BH;
    int nbq, nbk, topk;
    int32_t* order;
    const int32_t* idx_err;
};
hipError_t do_reverse(const RevArgs& r, hipStream_t st) {
    return aq::launch_reverse_index(r.idx, r.q_list, r.q_count, r.BH, r.nbq, r.nbk, r.topk, r.order,
                                    r.idx_err, st);
}

int run_fq(bool axis_d, bool quant, const aq::FqArgs& a, hipStream_t st, const char* what) {
    if (axis_d)
        return launch(K_FQ_D, st, quant ? thunk<aq::FqArgs, do_fq_d_q> : thunk<aq::FqArgs, do_fq_d_c>,
                      &a, what);
    return launch(K_FQ_N, st, quant ? thunk<aq::FqArgs, do_fq_n_q> : thunk<aq::FqArgs, do_fq_n_c>,
                  &a, what);
}

int run_transpose(const uint16_t* src, uint16_t* dst, int64_t BH, int64_t Npad, int64_t D,
                  bool perm, hipStream_t st, const char* what, bool to_f16 = false) {
    const TransposeArgs t{src, dst, BH, (int)Npad, (int)D, perm, to_f16};
    return launch(K_TRANSPOSE, st, thunk<TransposeArgs, do_transpose>, &t, what);
}

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

struct Strides {
    int64_t b, h, n;
};

Strides resolve(const attnqat_strides& s, int64_t H, int64_t N, int64_t D) {
    if (s.b == 0 && s.h == 0 && s.n == 0) return {H * N * D, N * D, D};
    return {s.b, s.h, s.n};
}

// Byte range [lo, hi) touched by a [B,H,N,D] tensor with strides s (elem bytes eb).
struct Range {
    uintptr_t lo, hi;
};

Range extent(const void* p, const Strides& s, int64_t B, int64_t H, int64_t N, int64_t D, int eb) {
    const uintptr_t base = (uintptr_t)p;
    const int64_t last = (B - 1) * s.b + (H - 1) * s.h + (N - 1) * s.n + (D - 1);
    return {base, base + (uintptr_t)((last + 1) * eb)};
}

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

int check_tensor(const char* name, const void* p, const Strides& s, int64_t H, int64_t N,
                 int64_t D) {
    if (!p) return fail(ATTNQAT_E_INVALID, "%s is NULL", name);
    if (s.b < 0 || s.h < 0 || s.n < 0)
        return fail(ATTNQAT_E_INVALID, "%s has a negative stride", name);
    if (((uintptr_t)p) % 16)
        return fail(ATTNQAT_E_MISALIGNED, "%s is not 16-byte aligned", name);
    if (s.b % 8 || s.h % 8 || s.n % 8)
        return fail(ATTNQAT_E_MISALIGNED, "%s strides (%lld, %lld, %lld) are not multiples of 8",
                    name, (long long)s.b, (long long)s.h, (long long)s.n);
    if (s.n < D && N > 1) return fail(ATTNQAT_E_INVALID, "%s rows overlap (stride_n < D)", name);
    (void)H;
    return ATTNQAT_OK;
}

// Longest sequence (query or key tokens) the attention entry points accept.
constexpr int64_t kMaxTokens = ATTNQAT_MAX_TOKENS;
static_assert(kMaxTokens * 128 * 2 < (int64_t(1) << 31), "32-bit tile offsets");

struct Plan {
    int64_t B, H, BH, Nq, Nk, D, Nq_pad, Nk_pad;
    Strides q, k, v, o, dout, dq, dk, dv;
    bool sparse;
    int nbq, nbk;
    bool rowmax_out;  // p_mode is ATTNQAT_P_ROWMAX: the forward writes the row maxima
    bool rowmax;      // ... and P is quantized: passes 2 and dK/dV use them
    bool f16_pv;      // forward P V on fp16 operands (V^T stored as fp16)
    size_t q_region;  // dense: bytes of the dQ partial sums (0: no split)
    size_t fo_region; // forward: bytes of the pass-2 partial sums (0: no split)
    int fo_rows;      // forward: queries per pass-2 workgroup (256; 128 with O_ste)
};

int validate_problem(const attnqat_problem* p, Plan& pl) {
    if (!p) return fail(ATTNQAT_E_INVALID, "problem is NULL");
    if (p->B < 1 || p->H < 1 || p->Nq < 1 || p->Nk < 1)
        return fail(ATTNQAT_E_INVALID, "sizes must be >= 1 (B=%lld H=%lld Nq=%lld Nk=%lld)",
                    (long long)p->B, (long long)p->H, (long long)p->Nq, (long long)p->Nk);
    if (p->D != 64 && p->D != 128)
        return fail(ATTNQAT_E_UNSUPPORTED, "head dimension %lld (supported: 64, 128)",
                    (long long)p->D);
    if (!std::isfinite(p->sm_scale) || !(p->sm_scale > 0.0f))
        return fail(ATTNQAT_E_INVALID, "sm_scale must be finite and > 0");
    if (p->quant_mask & ~ATTNQAT_QUANT_ALL)
        return fail(ATTNQAT_E_INVALID, "unknown quant_mask bits 0x%x", p->quant_mask);
    // the tile copies form 32-bit byte offsets of up to 128 rows of a
    // transposed [D][N] operand: 128 x N x 2 bytes must stay below 2^31
    if (p->Nq > kMaxTokens || p->Nk > kMaxTokens)
        return fail(ATTNQAT_E_UNSUPPORTED, "sequence length above %lld tokens (Nq=%lld Nk=%lld)",
                    (long long)kMaxTokens, (long long)p->Nq, (long long)p->Nk);
    // (batch, head) pairs index the second grid dimension of every kernel
    if (p->B * p->H > 65535)
        return fail(ATTNQAT_E_UNSUPPORTED, "B * H = %lld exceeds 65535",
                    (long long)(p->B * p->H));
    pl.B = p->B;
    pl.H = p->H;
    pl.BH = p->B * p->H;
    pl.Nq = p->Nq;
    pl.Nk = p->Nk;
    pl.D = p->D;
    pl.Nq_pad = round_up(p->Nq, aq::kTileN);
    pl.Nk_pad = round_up(p->Nk, aq::kTileN);
    pl.q = resolve(p->q, p->H, p->Nq, p->D);
    pl.k = resolve(p->k, p->H, p->Nk, p->D);
    pl.v = resolve(p->v, p->H, p->Nk, p->D);
    pl.o = resolve(p->o, p->H, p->Nq, p->D);
    pl.dout = resolve(p->dout, p->H, p->Nq, p->D);
    pl.dq = resolve(p->dq, p->H, p->Nq, p->D);
    pl.dk = resolve(p->dk, p->H, p->Nk, p->D);
    pl.dv = resolve(p->dv, p->H, p->Nk, p->D);
    if (p->p_mode != ATTNQAT_P_NORMALISED && p->p_mode != ATTNQAT_P_ROWMAX)
        return fail(ATTNQAT_E_INVALID, "unknown p_mode %u", p->p_mode);
    pl.rowmax_out = p->p_mode == ATTNQAT_P_ROWMAX;
    pl.rowmax = pl.rowmax_out && (p->quant_mask & ATTNQAT_QUANT_P);
    if (pl.rowmax_out) {
        if (!p->row_max) return fail(ATTNQAT_E_INVALID, "p_mode ATTNQAT_P_ROWMAX needs row_max");
        if (((uintptr_t)p->row_max) % 4)
            return fail(ATTNQAT_E_MISALIGNED, "row_max is not 4-byte aligned");
    }
    // P and V both quantized: the P V product runs on fp16 operands, which hold
    // NVFP4 values exactly, unless the unquantized P is multiplied too (o_ste)
    pl.f16_pv = (p->quant_mask & ATTNQAT_QUANT_P) && (p->quant_mask & ATTNQAT_QUANT_V) &&
                !p->o_ste;
    pl.sparse = p->kv_block_idx != nullptr;
    pl.nbq = pl.nbk = 0;
    if (pl.sparse) {
        if (p->block_tokens != 128)
            return fail(ATTNQAT_E_UNSUPPORTED, "block_tokens must be 128 (got %d)", p->block_tokens);
        pl.nbq = (int)((p->Nq + 127) / 128);
        pl.nbk = (int)((p->Nk + 127) / 128);
        if (p->topk < 1 || p->topk > pl.nbk)
            return fail(ATTNQAT_E_INVALID, "topk %d outside [1, %d]", p->topk, pl.nbk);
        if (pl.nbq > 1024 || pl.nbk > 1024)
            return fail(ATTNQAT_E_UNSUPPORTED, "block-sparse attention supports at most 1024 "
                        "blocks of 128 tokens per sequence");
        if (((uintptr_t)p->kv_block_idx) % 4)
            return fail(ATTNQAT_E_MISALIGNED, "kv_block_idx is not 4-byte aligned");
    }
    // dense dQ and the dense producer/consumer pass 2 (P quantized) run one
    // workgroup per 256-query block (128 for pass 2 with O_ste) in rounds of
    // one per compute unit; the planned split of the last round sizes their
    // partial regions: two slots of 256 x D fp32 per last-round workgroup (a
    // pass-2 slot with O_ste holds O and O_ste of 128 queries)
    const int64_t nkt = (pl.Nk + 63) / 64;
    const StreamSplit sq = stream_split(pl.BH * ((pl.Nq + 255) / 256), nkt, aq::kPlanCus);
    pl.q_region = pl.sparse ? 0 : (size_t)(2 * sq.chunks) * 256 * pl.D * 4;
    pl.fo_rows = p->o_ste ? 128 : 256;
    const StreamSplit sf =
        stream_split(pl.BH * ((pl.Nq + pl.fo_rows - 1) / pl.fo_rows), nkt, aq::kPlanCus);
    pl.fo_region = (!pl.sparse && (p->quant_mask & ATTNQAT_QUANT_P))
                       ? (size_t)(2 * sf.chunks) * 256 * pl.D * 4 : 0;
    return ATTNQAT_OK;
}

// Last-round split of dense dQ or forward pass 2 (blocks of `rows` queries)
// on the current device, or none when it does not fit the planned region of
// `region` bytes.
void query_split(const Plan& pl, int rows, size_t region, int& full, int& chunk, int& chunks) {
    const int64_t nqw = pl.BH * ((pl.Nq + rows - 1) / rows);
    full = (int)nqw;
    chunk = chunks = 0;
    if (region == 0) return;
    int cus = device_cus();
    if (cus > aq::kMaxDkdvSplit + 1) cus = aq::kMaxDkdvSplit + 1;
    const StreamSplit s = stream_split(nqw, (pl.Nk + 63) / 64, cus);
    if (!s.chunk || (size_t)(2 * s.chunks) * 256 * pl.D * 4 > region) return;
    full = (int)s.full;
    chunk = (int)s.chunk;
    chunks = (int)s.chunks;
}

// Workspace layout (bytes, each region 256-byte aligned).
struct Layout {
    size_t flag, qw, kw, vw, kt, vt, dow, lse2, delta, qlist, qcount, korder, dowkv, lse2kv,
        deltakv, dkdvpart, dkdvpart_bytes, fopart, total;
};

Layout layout(const Plan& pl, bool bwd) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    const size_t qb = (size_t)pl.BH * pl.Nq_pad * pl.D * 2;
    const size_t kb = (size_t)pl.BH * pl.Nk_pad * pl.D * 2;
    L.flag = take(256);  // block-index check: flag word at offset 0, then 63 partial words
    L.qw = take(qb);
    L.kw = take(kb);
    if (bwd) {
        L.vw = take(kb);
        if (!pl.sparse) L.kt = take(kb);
        L.dow = take(qb);
        L.lse2 = take((size_t)pl.BH * pl.Nq_pad * 4);
        L.delta = take((size_t)pl.BH * pl.Nq_pad * 4);
        if (pl.sparse) {
            L.qlist = take((size_t)pl.BH * pl.nbk * pl.nbq * 4);
            L.qcount = take((size_t)pl.BH * pl.nbk * 4);
            L.korder = take((size_t)pl.BH * pl.nbk * 4);
        }
        if (!pl.sparse) {
            // partial sums of the key blocks dK/dV splits ([part][2 x 128 rows]
            // per block), then of the query blocks dQ splits ([part][256 rows])
            const int64_t nkb = pl.BH * ((pl.Nk + 127) / 128);
            const int64_t ns = nkb < aq::kMaxDkdvSplit ? nkb : aq::kMaxDkdvSplit;
            const size_t kv = (size_t)ns * aq::kMaxDkdvParts * 256 * pl.D * 4;
            L.dkdvpart_bytes = kv > pl.q_region ? kv : pl.q_region;
            L.dkdvpart = take(L.dkdvpart_bytes);
        }
        if (pl.rowmax) {  // dK/dV inputs of the row-max-relative variant
            L.dowkv = take(qb);
            L.lse2kv = take((size_t)pl.BH * pl.Nq_pad * 4);
            L.deltakv = take((size_t)pl.BH * pl.Nq_pad * 4);
        }
    } else {
        L.vt = take(kb);  // Vq^T only: the forward kernels read V transposed
        if (pl.fo_region) L.fopart = take(pl.fo_region);
    }
    L.total = off;
    return L;
}

aq::FqArgs fq_args(const void* x, const Strides& xs, void* y, const Strides& ys, uint8_t* codes,
                   int64_t BH, int64_t H, int64_t N, int64_t Nout, int64_t D) {
    aq::FqArgs a{};
    a.x = (const uint16_t*)x;
    a.xsb = xs.b;
    a.xsh = xs.h;
    a.xsn = xs.n;
    a.y = (uint16_t*)y;
    a.ysb = ys.b;
    a.ysh = ys.h;
    a.ysn = ys.n;
    a.codes = codes;
    a.BH = BH;
    a.H = H;
    a.N = N;
    a.Nout = Nout;
    a.D = (int)D;
    return a;
}


// Quantize (or copy) q, k, v into the padded workspace operands.
int prepare_operands(const Plan& pl, uint32_t mask, const void* q, const void* k, const void* v,
                     char* ws, const Layout& L, bool bwd, hipStream_t st) {
    const Strides wq{pl.H * pl.Nq_pad * pl.D, pl.Nq_pad * pl.D, pl.D};
    const Strides wk{pl.H * pl.Nk_pad * pl.D, pl.Nk_pad * pl.D, pl.D};
    int rc;
    rc = run_fq(true, mask & ATTNQAT_QUANT_Q,
                fq_args(q, pl.q, ws + L.qw, wq, nullptr, pl.BH, pl.H, pl.Nq, pl.Nq_pad, pl.D), st,
                "fake-quant Q");
    if (rc) return rc;
    rc = run_fq(true, mask & ATTNQAT_QUANT_K,
                fq_args(k, pl.k, ws + L.kw, wk, nullptr, pl.BH, pl.H, pl.Nk, pl.Nk_pad, pl.D), st,
                "fake-quant K");
    if (rc) return rc;
    if (!bwd) {
        // the forward reads V only as V^T: quantize and transpose in one pass
        const Strides wt{pl.H * pl.D * pl.Nk_pad, pl.D * pl.Nk_pad, 0};
        const FqtArgs t{fq_args(v, pl.v, ws + L.vt, wt, nullptr, pl.BH, pl.H, pl.Nk, pl.Nk_pad, pl.D),
                        (mask & ATTNQAT_QUANT_V) != 0, pl.f16_pv};
        return launch(K_FQ_N, st, thunk<FqtArgs, do_fq_nt>, &t, "fake-quant and transpose V");
    }
    rc = run_fq(false, mask & ATTNQAT_QUANT_V,
                fq_args(v, pl.v, ws + L.vw, wk, nullptr, pl.BH, pl.H, pl.Nk, pl.Nk_pad, pl.D), st,
                "fake-quant V");
    if (rc) return rc;
    // the permuted K^T serves the dense dQ kernel only (the block-sparse one
    // reads K^T operands from its K tiles)
    if (pl.sparse) return ATTNQAT_OK;
    return run_transpose((const uint16_t*)(ws + L.kw), (uint16_t*)(ws + L.kt), pl.BH, pl.Nk_pad,
                         pl.D, true, st, "transpose K");
}

aq::AttnArgs attn_args(const attnqat_problem* p, const Plan& pl, char* ws, const Layout& L) {
    aq::AttnArgs a{};
    a.Qw = (const uint16_t*)(ws + L.qw);
    a.Kw = (const uint16_t*)(ws + L.kw);
    a.Vw = L.vw ? (const uint16_t*)(ws + L.vw) : nullptr;  // offset 0 is the flag word
    a.H = pl.H;
    a.Nq = (int)pl.Nq;
    a.Nk = (int)pl.Nk;
    a.Nq_pad = (int)pl.Nq_pad;
    a.Nk_pad = (int)pl.Nk_pad;
    a.BH = (int)pl.BH;
    a.sm_scale = p->sm_scale;
    a.c = p->sm_scale * aq::kLog2e;
    a.quant_p = (p->quant_mask & ATTNQAT_QUANT_P) ? 1 : 0;
    a.pv_f16 = pl.f16_pv ? 1 : 0;
    if (pl.sparse) {
        a.kv_idx = p->kv_block_idx;
        a.idx_err = (const int32_t*)(ws + L.flag);
        a.topk = p->topk;
        a.nbq = pl.nbq;
        a.nbk = pl.nbk;
    }
    return a;
}

// Block-sparse calls: check the caller's index on the device first; the
// sparse kernels skip their work when it fails.
struct CheckArgs {
    const int32_t* idx;
    int64_t rows;
    int topk, nbk;
    int32_t* flag;
};
hipError_t do_check(const CheckArgs& c, hipStream_t st) {
    return aq::launch_check_index(c.idx, c.rows, c.topk, c.nbk, c.flag, st);
}
int check_index(const attnqat_problem* p, const Plan& pl, char* ws, const Layout& L,
                hipStream_t st) {
    const CheckArgs c{p->kv_block_idx, pl.BH * pl.nbq, p->topk, pl.nbk, (int32_t*)(ws + L.flag)};
    return launch(K_CHECK_INDEX, st, thunk<CheckArgs, do_check>, &c, "block index check");
}

// ... and after the call, overwrite its outputs with NaN if the check failed.
void poison_add(aq::PoisonArgs& a, void* t, const Strides& s, int64_t N) {
    a.t[a.nt] = (uint16_t*)t;
    a.sb[a.nt] = s.b;
    a.sh[a.nt] = s.h;
    a.sn[a.nt] = s.n;
    a.N[a.nt] = N;
    ++a.nt;
}
void poison_add_f32(aq::PoisonArgs& a, float* f, int64_t n) {
    a.f[a.nf] = f;
    a.fn[a.nf] = n;
    ++a.nf;
}
int poison(const aq::PoisonArgs& a, hipStream_t st) {
    return launch(K_POISON, st, thunk<aq::PoisonArgs, aq::launch_poison_outputs>, &a,
                  "NaN fill after a failed index check");
}

}  // namespace

extern "C" {

int attnqat_abi_version(void) { return ATTNQAT_ABI_VERSION; }

const char* attnqat_status_string(int status) {
    switch (status) {
        case ATTNQAT_OK: return "ok";
        case ATTNQAT_E_INVALID: return "invalid argument";
        case ATTNQAT_E_UNSUPPORTED: return "unsupported configuration or device";
        case ATTNQAT_E_MISALIGNED: return "misaligned pointer or stride";
        case ATTNQAT_E_WORKSPACE: return "workspace missing or too small";
        case ATTNQAT_E_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* attnqat_last_error(void) { return g_last_error.c_str(); }

int attnqat_fakequant_nvfp4(const void* x, attnqat_strides xs, void* y, attnqat_strides ys,
                            uint8_t* scale_codes, int64_t B, int64_t H, int64_t N, int64_t D,
                            int group_axis, void* stream) {
    if (B < 1 || H < 1 || N < 1 || D < 1)
        return fail(ATTNQAT_E_INVALID, "sizes must be >= 1");
    if (group_axis != ATTNQAT_AXIS_D && group_axis != ATTNQAT_AXIS_N)
        return fail(ATTNQAT_E_INVALID, "group_axis must be ATTNQAT_AXIS_D or ATTNQAT_AXIS_N");
    if (D > 1024 || (group_axis == ATTNQAT_AXIS_D ? D % 16 : D % 8))
        return fail(ATTNQAT_E_UNSUPPORTED, "D=%lld unsupported for this axis", (long long)D);
    if (N > (int64_t)1 << 40 || B * H > (int64_t)1 << 31)
        return fail(ATTNQAT_E_INVALID, "sizes too large");
    const Strides sx = resolve(xs, H, N, D), sy = resolve(ys, H, N, D);
    int rc = check_tensor("x", x, sx, H, N, D);
    if (rc) return rc;
    rc = check_tensor("y", y, sy, H, N, D);
    if (rc) return rc;
    if (overlaps(extent(x, sx, B, H, N, D, 2), extent(y, sy, B, H, N, D, 2)))
        return fail(ATTNQAT_E_INVALID, "y overlaps x");
    if (scale_codes) {
        const int64_t nc = group_axis == ATTNQAT_AXIS_D ? B * H * N * (D / 16)
                                                        : B * H * ((N + 15) / 16) * D;
        const Range rc_ = {(uintptr_t)scale_codes, (uintptr_t)scale_codes + (uintptr_t)nc};
        if (overlaps(rc_, extent(x, sx, B, H, N, D, 2)) || overlaps(rc_, extent(y, sy, B, H, N, D, 2)))
            return fail(ATTNQAT_E_INVALID, "scale_codes overlaps x or y");
    }
    rc = check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    const aq::FqArgs a = fq_args(x, sx, y, sy, scale_codes, B * H, H, N, N, D);
    rc = run_fq(group_axis == ATTNQAT_AXIS_D, true, a, st, "fake-quant launch");
    return rc ? rc : ok();
}

size_t attnqat_fwd_workspace_bytes(const attnqat_problem* p) {
    Plan pl;
    if (validate_problem(p, pl)) return 0;
    return layout(pl, false).total;
}

size_t attnqat_bwd_workspace_bytes(const attnqat_problem* p) {
    Plan pl;
    if (validate_problem(p, pl)) return 0;
    return layout(pl, true).total;
}

int attnqat_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v, void* o,
                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    Plan pl;
    int rc = validate_problem(p, pl);
    if (rc) return rc;
    if ((rc = check_tensor("q", q, pl.q, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("k", k, pl.k, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("v", v, pl.v, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("o", o, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if (!lse) return fail(ATTNQAT_E_INVALID, "lse is NULL");
    if (((uintptr_t)lse) % 4) return fail(ATTNQAT_E_MISALIGNED, "lse is not 4-byte aligned");
    const Layout L = layout(pl, false);
    if (!workspace || workspace_bytes < L.total)
        return fail(ATTNQAT_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256)
        return fail(ATTNQAT_E_MISALIGNED, "workspace is not 256-byte aligned");
    const Range ro = extent(o, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2);
    const Range rl = {(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(pl.BH * pl.Nq * 4)};
    const Range rw = {(uintptr_t)workspace, (uintptr_t)workspace + L.total};
    const Range rm = pl.rowmax_out ? Range{(uintptr_t)p->row_max,
                                           (uintptr_t)p->row_max + (uintptr_t)(pl.BH * pl.Nq * 4)}
                                   : Range{0, 0};
    if (p->o_ste && (rc = check_tensor("o_ste", p->o_ste, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    const Range rs = p->o_ste ? extent(p->o_ste, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2) : Range{0, 0};
    const Range ins[3] = {extent(q, pl.q, pl.B, pl.H, pl.Nq, pl.D, 2),
                          extent(k, pl.k, pl.B, pl.H, pl.Nk, pl.D, 2),
                          extent(v, pl.v, pl.B, pl.H, pl.Nk, pl.D, 2)};
    for (const Range& r : ins)
        if (overlaps(r, ro) || overlaps(r, rl) || overlaps(r, rw) || overlaps(r, rm) ||
            overlaps(r, rs))
            return fail(ATTNQAT_E_INVALID, "an output or the workspace overlaps an input");
    if (overlaps(ro, rl) || overlaps(ro, rw) || overlaps(rl, rw) || overlaps(rm, ro) ||
        overlaps(rm, rl) || overlaps(rm, rw) || overlaps(rs, ro) || overlaps(rs, rl) ||
        overlaps(rs, rw) || overlaps(rs, rm))
        return fail(ATTNQAT_E_INVALID, "outputs overlap each other or the workspace");
    if ((rc = check_device())) return rc;

    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    if (pl.sparse && (rc = check_index(p, pl, ws, L, st))) return rc;
    if ((rc = prepare_operands(pl, p->quant_mask, q, k, v, ws, L, false, st))) return rc;
    aq::AttnArgs a = attn_args(p, pl, ws, L);
    a.Vt = (const uint16_t*)(ws + L.vt);
    a.lse_out = lse;
    a.row_max_out = pl.rowmax_out ? p->row_max : nullptr;
    a.o_ste = (uint16_t*)p->o_ste;
    a.row_max = pl.rowmax ? p->row_max : nullptr;
    a.lse = lse;
    a.o = (uint16_t*)o;
    a.osb = pl.o.b;
    a.osh = pl.o.h;
    a.osn = pl.o.n;
    if (!pl.sparse) {
        query_split(pl, pl.fo_rows, pl.fo_region, a.fo_full, a.fo_chunk, a.fo_chunks);
        a.fo_part = (float*)(ws + L.fopart);
    }
    const DimArgs da{a, (int)pl.D};
    if (!(p->quant_mask & ATTNQAT_QUANT_P)) {
        // no P quantizer: nothing needs the final LSE before P V
        if ((rc = launch(K_FWD_SINGLE, st, thunk<DimArgs, do_fwd_single>, &da, "forward")))
            return rc;
    } else {
        if ((rc = launch(K_FWD_LSE, st, thunk<DimArgs, do_fwd_lse>, &da, "forward pass 1")))
            return rc;
        if ((rc = launch(K_FWD_OUT, st, thunk<DimArgs, do_fwd_out>, &da, "forward pass 2")))
            return rc;
    }
    if (pl.sparse) {
        aq::PoisonArgs pa{};
        pa.flag = a.idx_err;
        pa.BH = pl.BH;
        pa.H = pl.H;
        pa.D = (int)pl.D;
        poison_add(pa, o, pl.o, pl.Nq);
        if (p->o_ste) poison_add(pa, p->o_ste, pl.o, pl.Nq);
        poison_add_f32(pa, lse, pl.BH * pl.Nq);
        if (pl.rowmax_out) poison_add_f32(pa, p->row_max, pl.BH * pl.Nq);
        if ((rc = poison(pa, st))) return rc;
    }
    return ok();
}

int attnqat_fwd_noalloc(const attnqat_problem* p, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* stream) {
    Plan pl;
    int rc = validate_problem(p, pl);
    if (rc) return rc;
    const size_t need = layout(pl, false).total;
    if (need > aq::kNoAllocScratchBytes)
        return fail(ATTNQAT_E_UNSUPPORTED,
                    "attnqat_fwd_noalloc: this problem needs %zu bytes of scratch; the fixed "
                    "device buffer holds %zu (use attnqat_fwd with a workspace)",
                    need, aq::kNoAllocScratchBytes);
    if ((rc = check_device())) return rc;
    int dev = 0;
    if ((rc = hip_check(hipGetDevice(&dev), "hipGetDevice"))) return rc;
    void* ws = nullptr;
    if ((rc = hip_check(aq::noalloc_scratch(dev, &ws), "hipGetSymbolAddress of the scratch")))
        return rc;
    return attnqat_fwd(p, q, k, v, o, lse, ws, aq::kNoAllocScratchBytes, stream);
}

int attnqat_bwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, void* stream) {
    Plan pl;
    int rc = validate_problem(p, pl);
    if (rc) return rc;
    if ((rc = check_tensor("q", q, pl.q, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("k", k, pl.k, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("v", v, pl.v, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("o", o, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("dout", dout, pl.dout, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("dq", dq, pl.dq, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("dk", dk, pl.dk, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("dv", dv, pl.dv, pl.H, pl.Nk, pl.D))) return rc;
    if (!lse) return fail(ATTNQAT_E_INVALID, "lse is NULL");
    if (((uintptr_t)lse) % 4) return fail(ATTNQAT_E_MISALIGNED, "lse is not 4-byte aligned");
    const Layout L = layout(pl, true);
    if (!workspace || workspace_bytes < L.total)
        return fail(ATTNQAT_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256)
        return fail(ATTNQAT_E_MISALIGNED, "workspace is not 256-byte aligned");
    const Range outs[4] = {extent(dq, pl.dq, pl.B, pl.H, pl.Nq, pl.D, 2),
                           extent(dk, pl.dk, pl.B, pl.H, pl.Nk, pl.D, 2),
                           extent(dv, pl.dv, pl.B, pl.H, pl.Nk, pl.D, 2),
                           {(uintptr_t)workspace, (uintptr_t)workspace + L.total}};
    const Range ins[7] = {
        extent(q, pl.q, pl.B, pl.H, pl.Nq, pl.D, 2),
        extent(k, pl.k, pl.B, pl.H, pl.Nk, pl.D, 2),
        extent(v, pl.v, pl.B, pl.H, pl.Nk, pl.D, 2),
        extent(o, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2),
        extent(dout, pl.dout, pl.B, pl.H, pl.Nq, pl.D, 2),
        {(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(pl.BH * pl.Nq * 4)},
        pl.rowmax ? Range{(uintptr_t)p->row_max, (uintptr_t)p->row_max + (uintptr_t)(pl.BH * pl.Nq * 4)}
                  : Range{0, 0}};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlaps(outs[i], ins[j]))
                return fail(ATTNQAT_E_INVALID, "an output or the workspace overlaps an input");
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(ATTNQAT_E_INVALID, "outputs overlap each other or the workspace");
    }
    if ((rc = check_device())) return rc;

    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    if (pl.sparse && (rc = check_index(p, pl, ws, L, st))) return rc;
    if ((rc = prepare_operands(pl, p->quant_mask, q, k, v, ws, L, true, st))) return rc;
    aq::PreArgs pa{};
    pa.o = (const uint16_t*)o;
    pa.osb = pl.o.b;
    pa.osh = pl.o.h;
    pa.osn = pl.o.n;
    pa.dout = (const uint16_t*)dout;
    pa.dsb = pl.dout.b;
    pa.dsh = pl.dout.h;
    pa.dsn = pl.dout.n;
    pa.lse = lse;
    pa.delta = (float*)(ws + L.delta);
    pa.lse2 = (float*)(ws + L.lse2);
    pa.dOw = (uint16_t*)(ws + L.dow);
    if (pl.rowmax) {
        pa.row_max = p->row_max;
        pa.dOw_kv = (uint16_t*)(ws + L.dowkv);
        pa.lse2_kv = (float*)(ws + L.lse2kv);
        pa.delta_kv = (float*)(ws + L.deltakv);
    }
    pa.BH = pl.BH;
    pa.H = pl.H;
    pa.Nq = pl.Nq;
    pa.Nq_pad = pl.Nq_pad;
    pa.D = (int)pl.D;
    if ((rc = launch(K_BWD_PRE, st, thunk<aq::PreArgs, aq::launch_bwd_pre>, &pa,
                     "backward preprocess")))
        return rc;
    aq::AttnArgs a = attn_args(p, pl, ws, L);
    a.Kt = pl.sparse ? nullptr : (const uint16_t*)(ws + L.kt);
    a.dOw = (const uint16_t*)(ws + L.dow);
    a.lse2 = (const float*)(ws + L.lse2);
    a.delta = (const float*)(ws + L.delta);
    a.dq = (uint16_t*)dq;
    a.dqsb = pl.dq.b;
    a.dqsh = pl.dq.h;
    a.dqsn = pl.dq.n;
    a.dk = (uint16_t*)dk;
    a.dksb = pl.dk.b;
    a.dksh = pl.dk.h;
    a.dksn = pl.dk.n;
    a.dv = (uint16_t*)dv;
    a.dvsb = pl.dv.b;
    a.dvsh = pl.dv.h;
    a.dvsn = pl.dv.n;
    if (pl.sparse) {
        a.q_list = (const int32_t*)(ws + L.qlist);
        a.q_count = (const int32_t*)(ws + L.qcount);
        a.kv_order = (const int32_t*)(ws + L.korder);
        const RevArgs ra{p->kv_block_idx, (int32_t*)(ws + L.qlist), (int32_t*)(ws + L.qcount),
                         pl.BH, pl.nbq, pl.nbk, p->topk, (int32_t*)(ws + L.korder),
                         a.idx_err};
        if ((rc = launch(K_REVERSE_INDEX, st, thunk<RevArgs, do_reverse>, &ra,
                         "reverse block index")))
            return rc;
    }
    if (!pl.sparse) {
        // dense dK/dV: one workgroup per key block runs in rounds of one
        // workgroup per compute unit; the F blocks of the last, partial round
        // are split into P parts along the queries (P <= 4, the one that
        // minimises the last round's length ceil(F P / CUs) / P)
        a.nbk = (int)((pl.Nk + 127) / 128);
        const int64_t nkb = pl.BH * a.nbk;
        int cus = device_cus();
        if (cus > aq::kMaxDkdvSplit + 1) cus = aq::kMaxDkdvSplit + 1;
        const int64_t F = nkb % cus;
        const int64_t nt = (pl.Nq + 63) / 64;  // query tiles: a part has at least one
        const int P = split_parts(F, cus, nt);
        a.dkdv_parts = P;
        a.dkdv_full = (int)(P > 1 ? nkb - F : nkb);
        a.dkdv_part = (float*)(ws + L.dkdvpart);
        // dense dQ: one workgroup per 256-query block, its last round shared
        // out along the key tiles, partial sums in the same region
        query_split(pl, 256, L.dkdvpart_bytes, a.dq_full, a.dq_chunk, a.dq_chunks);
        a.dq_part = (float*)(ws + L.dkdvpart);
    }
    const DimArgs da{a, (int)pl.D};
    // row-max-relative variant: dK/dV quantizes exp(S - m) and takes dO and Dl
    // scaled by 1/l (the backward preprocess wrote them)
    aq::AttnArgs akv = a;
    if (pl.rowmax) {
        akv.dOw = (const uint16_t*)(ws + L.dowkv);
        akv.lse2 = (const float*)(ws + L.lse2kv);
        akv.delta = (const float*)(ws + L.deltakv);
    }
    const DimArgs dkv{akv, (int)pl.D};
    if ((rc = launch(K_BWD_DKDV, st, thunk<DimArgs, do_bwd_dkdv>, &dkv, "backward dK/dV")))
        return rc;
    if ((rc = launch(K_BWD_DQ, st, thunk<DimArgs, do_bwd_dq>, &da, "backward dQ"))) return rc;
    if (pl.sparse) {
        aq::PoisonArgs pz{};
        pz.flag = a.idx_err;
        pz.BH = pl.BH;
        pz.H = pl.H;
        pz.D = (int)pl.D;
        poison_add(pz, dq, pl.dq, pl.Nq);
        poison_add(pz, dk, pl.dk, pl.Nk);
        poison_add(pz, dv, pl.dv, pl.Nk);
        if ((rc = poison(pz, st))) return rc;
    }
    return ok();
}

int attnqat_block_idx_status(const void* workspace, int* invalid, void* stream) {
    if (!workspace || !invalid) return fail(ATTNQAT_E_INVALID, "workspace or invalid is NULL");
    if (((uintptr_t)workspace) % 256)
        return fail(ATTNQAT_E_MISALIGNED, "workspace is not 256-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    int32_t flag = 0;
    if ((rc = hip_check(hipMemcpyAsync(&flag, workspace, 4, hipMemcpyDeviceToHost, st),
                        "hipMemcpyAsync")))
        return rc;
    if ((rc = hip_check(hipStreamSynchronize(st), "hipStreamSynchronize"))) return rc;
    *invalid = flag != 0;
    return ok();
}

int attnqat_effective_topk(int64_t num_blocks, double sparsity) {
    if (num_blocks < 1 || num_blocks > (int64_t)1 << 30 || !(sparsity >= 0.0 && sparsity <= 1.0))
        return -fail(ATTNQAT_E_INVALID, "num_blocks must be >= 1 and sparsity in [0, 1]");
    const double kept = std::ceil((1.0 - sparsity) * (double)num_blocks);
    int64_t k = (int64_t)kept;
    if (k > num_blocks) k = num_blocks;
    if (k < 1) k = 1;
    ok();
    return (int)k;
}

size_t attnqat_block_select_workspace_bytes(const attnqat_problem* p) {
    if (!p || p->B < 1 || p->H < 1 || p->Nq < 1 || p->Nk < 1 || p->D < 1 || p->block_tokens < 1)
        return 0;
    const int64_t nbq = (p->Nq + p->block_tokens - 1) / p->block_tokens;
    const int64_t nbk = (p->Nk + p->block_tokens - 1) / p->block_tokens;
    const size_t a = (size_t)(p->B * p->H * nbq * p->D * 2 + 255) / 256 * 256;
    const size_t b = (size_t)(p->B * p->H * nbk * p->D * 2 + 255) / 256 * 256;
    return a + b;
}

int attnqat_block_select(const attnqat_problem* p, const void* q, const void* k,
                         int32_t* kv_block_idx, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (!p) return fail(ATTNQAT_E_INVALID, "problem is NULL");
    if (p->B < 1 || p->H < 1 || p->Nq < 1 || p->Nk < 1)
        return fail(ATTNQAT_E_INVALID, "sizes must be >= 1");
    if (p->D != 64 && p->D != 128)
        return fail(ATTNQAT_E_UNSUPPORTED, "head dimension %lld (supported: 64, 128)",
                    (long long)p->D);
    if (p->B * p->H > 65535)
        return fail(ATTNQAT_E_UNSUPPORTED, "B * H = %lld exceeds 65535", (long long)(p->B * p->H));
    if (p->block_tokens < 1 || p->block_tokens > 4096)
        return fail(ATTNQAT_E_INVALID, "block_tokens %d outside [1, 4096]", p->block_tokens);
    const int64_t nbq = (p->Nq + p->block_tokens - 1) / p->block_tokens;
    const int64_t nbk = (p->Nk + p->block_tokens - 1) / p->block_tokens;
    if (nbk > 1024) return fail(ATTNQAT_E_UNSUPPORTED, "more than 1024 key blocks");
    if (p->topk < 1 || p->topk > nbk)
        return fail(ATTNQAT_E_INVALID, "topk %d outside [1, %lld]", p->topk, (long long)nbk);
    if (p->Nq > (1 << 30) || p->Nk > (1 << 30) || p->B * p->H > (1 << 30))
        return fail(ATTNQAT_E_INVALID, "sizes too large");
    // (batch, head) pairs index the second grid dimension of every kernel
    if (p->B * p->H > 65535)
        return fail(ATTNQAT_E_UNSUPPORTED, "B * H = %lld exceeds 65535",
                    (long long)(p->B * p->H));
    const Strides sq = resolve(p->q, p->H, p->Nq, p->D), sk = resolve(p->k, p->H, p->Nk, p->D);
    int rc;
    if ((rc = check_tensor("q", q, sq, p->H, p->Nq, p->D))) return rc;
    if ((rc = check_tensor("k", k, sk, p->H, p->Nk, p->D))) return rc;
    if (!kv_block_idx) return fail(ATTNQAT_E_INVALID, "kv_block_idx is NULL");
    if (((uintptr_t)kv_block_idx) % 4)
        return fail(ATTNQAT_E_MISALIGNED, "kv_block_idx is not 4-byte aligned");
    const size_t need = attnqat_block_select_workspace_bytes(p);
    if (!workspace || workspace_bytes < need)
        return fail(ATTNQAT_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256)
        return fail(ATTNQAT_E_MISALIGNED, "workspace is not 256-byte aligned");
    const Range ri = {(uintptr_t)kv_block_idx,
                      (uintptr_t)kv_block_idx + (uintptr_t)(p->B * p->H * nbq * p->topk * 4)};
    const Range rw = {(uintptr_t)workspace, (uintptr_t)workspace + need};
    const Range rq = extent(q, sq, p->B, p->H, p->Nq, p->D, 2);
    const Range rk = extent(k, sk, p->B, p->H, p->Nk, p->D, 2);
    if (overlaps(ri, rq) || overlaps(ri, rk) || overlaps(rw, rq) || overlaps(rw, rk) ||
        overlaps(ri, rw))
        return fail(ATTNQAT_E_INVALID, "kv_block_idx or the workspace overlaps an input");
    if ((rc = check_device())) return rc;
    aq::SelectArgs a{};
    a.q = (const uint16_t*)q;
    a.qsb = sq.b;
    a.qsh = sq.h;
    a.qsn = sq.n;
    a.k = (const uint16_t*)k;
    a.ksb = sk.b;
    a.ksh = sk.h;
    a.ksn = sk.n;
    const size_t qbar_bytes = (size_t)(p->B * p->H * nbq * p->D * 2 + 255) / 256 * 256;
    a.qbar = (uint16_t*)workspace;
    a.kbar = (uint16_t*)((char*)workspace + qbar_bytes);
    a.idx = kv_block_idx;
    a.BH = p->B * p->H;
    a.H = p->H;
    a.Nq = (int)p->Nq;
    a.Nk = (int)p->Nk;
    a.bt = p->block_tokens;
    a.nbq = (int)nbq;
    a.nbk = (int)nbk;
    a.topk = p->topk;
    a.D = (int)p->D;
    hipStream_t st = (hipStream_t)stream;
    if ((rc = launch(K_BLOCK_POOL, st, thunk<aq::SelectArgs, aq::launch_block_pool>, &a,
                     "block pooling")))
        return rc;
    if ((rc = launch(K_BLOCK_TOPK, st, thunk<aq::SelectArgs, aq::launch_block_topk>, &a,
                     "block top-k")))
        return rc;
    return ok();
}

// ---------------------------------------------------------------------------
// VSA coarse branch
namespace {

struct VsaLayout {
    size_t qbar, kbar, vbar, oc, lsec, doc, dcc, dqb, dkb, dvb, total;
};

VsaLayout vsa_layout(int64_t BH, int64_t nbq, int64_t nbk, int64_t D) {
    VsaLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    L.qbar = take((size_t)(BH * nbq * D * 2));
    L.kbar = take((size_t)(BH * nbk * D * 2));
    L.vbar = take((size_t)(BH * nbk * D * 2));
    L.oc = take((size_t)(BH * nbq * D * 4));
    L.lsec = take((size_t)(BH * nbq * 4));
    L.doc = take((size_t)(BH * nbq * D * 4));
    L.dcc = take((size_t)(BH * nbq * 4));
    L.dqb = take((size_t)(BH * nbq * D * 4));
    L.dkb = take((size_t)(BH * nbk * D * 4));
    L.dvb = take((size_t)(BH * nbk * D * 4));
    L.total = off;
    return L;
}

int vsa_plan(const attnqat_problem* p, Plan& pl, int64_t& nbq, int64_t& nbk, VsaLayout& L) {
    int rc = validate_problem(p, pl);
    if (rc) return rc;
    if (p->block_tokens != 128)
        return fail(ATTNQAT_E_UNSUPPORTED, "VSA blocks must be 128 tokens (got %d)", p->block_tokens);
    nbq = (pl.Nq + 127) / 128;
    nbk = (pl.Nk + 127) / 128;
    if (nbq > aq::kVsaMaxBlocks || nbk > aq::kVsaMaxBlocks)
        return fail(ATTNQAT_E_UNSUPPORTED, "VSA supports at most %d blocks per sequence",
                    aq::kVsaMaxBlocks);
    L = vsa_layout(pl.BH, nbq, nbk, pl.D);
    return ATTNQAT_OK;
}

aq::VsaArgs vsa_args(const attnqat_problem* p, const Plan& pl, int64_t nbq, int64_t nbk,
                     const VsaLayout& L, char* ws, const void* q, const void* k, const void* v,
                     const void* gate) {
    aq::VsaArgs a{};
    a.q = (const uint16_t*)q;
    a.qsb = pl.q.b;
    a.qsh = pl.q.h;
    a.qsn = pl.q.n;
    a.k = (const uint16_t*)k;
    a.ksb = pl.k.b;
    a.ksh = pl.k.h;
    a.ksn = pl.k.n;
    a.v = (const uint16_t*)v;
    a.vsb = pl.v.b;
    a.vsh = pl.v.h;
    a.vsn = pl.v.n;
    a.gate = (const uint16_t*)gate;
    a.osb = pl.o.b;
    a.osh = pl.o.h;
    a.osn = pl.o.n;
    a.qbar = (uint16_t*)(ws + L.qbar);
    a.kbar = (uint16_t*)(ws + L.kbar);
    a.vbar = (uint16_t*)(ws + L.vbar);
    a.oc = (float*)(ws + L.oc);
    a.lsec = (float*)(ws + L.lsec);
    a.doc = (float*)(ws + L.doc);
    a.dcc = (float*)(ws + L.dcc);
    a.dqb = (float*)(ws + L.dqb);
    a.dkb = (float*)(ws + L.dkb);
    a.dvb = (float*)(ws + L.dvb);
    a.BH = pl.BH;
    a.H = pl.H;
    a.Nq = (int)pl.Nq;
    a.Nk = (int)pl.Nk;
    a.bt = 128;
    a.nbq = (int)nbq;
    a.nbk = (int)nbk;
    a.D = (int)pl.D;
    a.sm_scale = p->sm_scale;
    return a;
}

int check_workspace(void* ws, size_t have, size_t need) {
    if (!ws || have < need)
        return fail(ATTNQAT_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                    ws ? have : (size_t)0);
    if (((uintptr_t)ws) % 256) return fail(ATTNQAT_E_MISALIGNED, "workspace is not 256-byte aligned");
    return ATTNQAT_OK;
}

// The coarse forward: block means, then the coarse attention rows.
int vsa_coarse(const aq::VsaArgs& a, hipStream_t st) {
    int rc;
    if ((rc = launch(K_VSA_POOL, st, thunk<aq::VsaArgs, aq::launch_vsa_pool>, &a, "VSA block means")))
        return rc;
    return launch(K_VSA_COARSE, st, thunk<aq::VsaArgs, aq::launch_vsa_coarse_fwd>, &a,
                  "VSA coarse attention");
}

}  // namespace

size_t attnqat_vsa_workspace_bytes(const attnqat_problem* p) {
    Plan pl;
    int64_t nbq, nbk;
    VsaLayout L;
    if (vsa_plan(p, pl, nbq, nbk, L)) return 0;
    return L.total;
}

int attnqat_vsa_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                    const void* gate, const void* o_fine, void* o, void* workspace,
                    size_t workspace_bytes, void* stream) {
    Plan pl;
    int64_t nbq, nbk;
    VsaLayout L;
    int rc = vsa_plan(p, pl, nbq, nbk, L);
    if (rc) return rc;
    if ((rc = check_tensor("q", q, pl.q, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("k", k, pl.k, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("v", v, pl.v, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("gate", gate, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("o_fine", o_fine, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("o", o, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, L.total))) return rc;
    const Range ins[5] = {extent(q, pl.q, pl.B, pl.H, pl.Nq, pl.D, 2),
                          extent(k, pl.k, pl.B, pl.H, pl.Nk, pl.D, 2),
                          extent(v, pl.v, pl.B, pl.H, pl.Nk, pl.D, 2),
                          extent(gate, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2),
                          extent(o_fine, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2)};
    const Range ro = extent(o, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2);
    const Range rw = {(uintptr_t)workspace, (uintptr_t)workspace + L.total};
    if (overlaps(ro, rw)) return fail(ATTNQAT_E_INVALID, "o overlaps the workspace");
    for (const Range& r : ins)
        if (overlaps(r, ro) || overlaps(r, rw))
            return fail(ATTNQAT_E_INVALID, "o or the workspace overlaps an input");
    if ((rc = check_device())) return rc;
    hipStream_t st = (hipStream_t)stream;
    aq::VsaArgs a = vsa_args(p, pl, nbq, nbk, L, (char*)workspace, q, k, v, gate);
    a.o_fine = (const uint16_t*)o_fine;
    a.o = (uint16_t*)o;
    if ((rc = vsa_coarse(a, st))) return rc;
    if ((rc = launch(K_VSA_COMBINE, st, thunk<aq::VsaArgs, aq::launch_vsa_combine>, &a,
                     "VSA gated combination")))
        return rc;
    return ok();
}

int attnqat_vsa_bwd(const attnqat_problem* p, const void* q, const void* k, const void* v,
                    const void* gate, const void* dout, void* dq, void* dk, void* dv,
                    void* dgate, void* workspace, size_t workspace_bytes, void* stream) {
    Plan pl;
    int64_t nbq, nbk;
    VsaLayout L;
    int rc = vsa_plan(p, pl, nbq, nbk, L);
    if (rc) return rc;
    if ((rc = check_tensor("q", q, pl.q, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("k", k, pl.k, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("v", v, pl.v, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("gate", gate, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("dout", dout, pl.dout, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("dq", dq, pl.dq, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("dk", dk, pl.dk, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("dv", dv, pl.dv, pl.H, pl.Nk, pl.D))) return rc;
    if (dgate && (rc = check_tensor("dgate", dgate, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, L.total))) return rc;
    const Range ins[5] = {extent(q, pl.q, pl.B, pl.H, pl.Nq, pl.D, 2),
                          extent(k, pl.k, pl.B, pl.H, pl.Nk, pl.D, 2),
                          extent(v, pl.v, pl.B, pl.H, pl.Nk, pl.D, 2),
                          extent(gate, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2),
                          extent(dout, pl.dout, pl.B, pl.H, pl.Nq, pl.D, 2)};
    const Range outs[5] = {extent(dq, pl.dq, pl.B, pl.H, pl.Nq, pl.D, 2),
                           extent(dk, pl.dk, pl.B, pl.H, pl.Nk, pl.D, 2),
                           extent(dv, pl.dv, pl.B, pl.H, pl.Nk, pl.D, 2),
                           dgate ? extent(dgate, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2) : Range{0, 0},
                           {(uintptr_t)workspace, (uintptr_t)workspace + L.total}};
    for (int i = 0; i < 5; ++i) {
        for (const Range& r : ins)
            if (overlaps(outs[i], r))
                return fail(ATTNQAT_E_INVALID, "an output or the workspace overlaps an input");
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(ATTNQAT_E_INVALID, "outputs overlap each other or the workspace");
    }
    if ((rc = check_device())) return rc;
    hipStream_t st = (hipStream_t)stream;
    aq::VsaArgs a = vsa_args(p, pl, nbq, nbk, L, (char*)workspace, q, k, v, gate);
    a.dout = (const uint16_t*)dout;
    a.dsb = pl.dout.b;
    a.dsh = pl.dout.h;
    a.dsn = pl.dout.n;
    a.dq = (uint16_t*)dq;
    a.dqsb = pl.dq.b;
    a.dqsh = pl.dq.h;
    a.dqsn = pl.dq.n;
    a.dk = (uint16_t*)dk;
    a.dksb = pl.dk.b;
    a.dksh = pl.dk.h;
    a.dksn = pl.dk.n;
    a.dv = (uint16_t*)dv;
    a.dvsb = pl.dv.b;
    a.dvsh = pl.dv.h;
    a.dvsn = pl.dv.n;
    a.dgate = (uint16_t*)dgate;
    if ((rc = vsa_coarse(a, st))) return rc;
    if ((rc = launch(K_VSA_GATE, st, thunk<aq::VsaArgs, aq::launch_vsa_gate_reduce>, &a,
                     "VSA gate reduction")))
        return rc;
    if ((rc = launch(K_VSA_COARSE_BWD, st, thunk<aq::VsaArgs, aq::launch_vsa_coarse_bwd>, &a,
                     "VSA coarse backward")))
        return rc;
    if ((rc = launch(K_VSA_GRAD_ADD, st, thunk<aq::VsaArgs, aq::launch_vsa_grad_add>, &a,
                     "VSA gradient broadcast")))
        return rc;
    return ok();
}

int attnqat_profile_enable(int on) {
    g_prof.on = on != 0;
    g_prof.used = 0;
    return ok();
}

int attnqat_profile_read(const char** names, double* total_ms, int* launches, int max_kinds) {
    double tot[K_NUM] = {0};
    int cnt[K_NUM] = {0};
    Profiler& P = g_prof;
    for (int i = 0; i < P.used; ++i) {
        hipError_t e = hipEventSynchronize(P.ev[2 * i + 1]);
        if (e != hipSuccess) {
            P.used = 0;
            return -fail(ATTNQAT_E_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
        }
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, P.ev[2 * i], P.ev[2 * i + 1]);
        if (e != hipSuccess) {
            P.used = 0;
            return -fail(ATTNQAT_E_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
        }
        tot[P.kind[i]] += ms;
        cnt[P.kind[i]] += 1;
    }
    P.used = 0;
    int n = 0;
    for (int k = 0; k < K_NUM && n < max_kinds; ++k) {
        if (!cnt[k]) continue;
        if (names) names[n] = kKindName[k];
        if (total_ms) total_ms[n] = tot[k];
        if (launches) launches[n] = cnt[k];
        ++n;
    }
    ok();
    return n;
}

// ---------------------------------------------------------------------------
// Real-FP4 (MXFP4) inference forward

}  // extern "C"

namespace {
struct MxLayout {
    size_t qm, qs, km, ks, vtm, vts, total;
};
MxLayout mx_layout(const Plan& pl) {
    MxLayout L{};
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t at = off;
        off += (n + 255) / 256 * 256;
        return at;
    };
    const size_t bh = (size_t)pl.BH, D = (size_t)pl.D;
    L.qm = take(bh * pl.Nq_pad * D / 2);
    L.qs = take(bh * pl.Nq_pad * D / 32);
    L.km = take(bh * pl.Nk_pad * D / 2);
    L.ks = take(bh * pl.Nk_pad * D / 32);
    L.vtm = take(bh * D * pl.Nk_pad / 2);
    L.vts = take(bh * D * pl.Nk_pad / 32);
    L.total = off;
    return L;
}
int mx_plan(const attnqat_problem* p, Plan& pl) {
    if (!p) return fail(ATTNQAT_E_INVALID, "problem is NULL");
    if (p->kv_block_idx)
        return fail(ATTNQAT_E_UNSUPPORTED, "the MXFP4 forward is dense: kv_block_idx must be NULL");
    if (p->o_ste)
        return fail(ATTNQAT_E_UNSUPPORTED, "the MXFP4 forward has no straight-through output");
    if (p->quant_mask != ATTNQAT_QUANT_ALL)
        return fail(ATTNQAT_E_UNSUPPORTED,
                    "the MXFP4 forward quantizes Q, K, V and P: quant_mask must be ATTNQAT_QUANT_ALL");
    attnqat_problem c = *p;  // P is always row-max relative here; p_mode and row_max are unused
    c.p_mode = ATTNQAT_P_NORMALISED;
    c.row_max = nullptr;
    return validate_problem(&c, pl);
}
}  // namespace

extern "C" {

size_t attnqat_mxfp4_fwd_workspace_bytes(const attnqat_problem* p) {
    Plan pl;
    if (mx_plan(p, pl)) return 0;
    return mx_layout(pl).total;
}

int attnqat_mxfp4_fwd(const attnqat_problem* p, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    Plan pl;
    int rc = mx_plan(p, pl);
    if (rc) return rc;
    if ((rc = check_tensor("q", q, pl.q, pl.H, pl.Nq, pl.D))) return rc;
    if ((rc = check_tensor("k", k, pl.k, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("v", v, pl.v, pl.H, pl.Nk, pl.D))) return rc;
    if ((rc = check_tensor("o", o, pl.o, pl.H, pl.Nq, pl.D))) return rc;
    if (!lse) return fail(ATTNQAT_E_INVALID, "lse is NULL");
    if (((uintptr_t)lse) % 4) return fail(ATTNQAT_E_MISALIGNED, "lse is not 4-byte aligned");
    const MxLayout L = mx_layout(pl);
    if (!workspace || workspace_bytes < L.total)
        return fail(ATTNQAT_E_WORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace) % 256)
        return fail(ATTNQAT_E_MISALIGNED, "workspace is not 256-byte aligned");
    const Range ro = extent(o, pl.o, pl.B, pl.H, pl.Nq, pl.D, 2);
    const Range rl = {(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(pl.BH * pl.Nq * 4)};
    const Range rw = {(uintptr_t)workspace, (uintptr_t)workspace + L.total};
    const Range ins[3] = {extent(q, pl.q, pl.B, pl.H, pl.Nq, pl.D, 2),
                          extent(k, pl.k, pl.B, pl.H, pl.Nk, pl.D, 2),
                          extent(v, pl.v, pl.B, pl.H, pl.Nk, pl.D, 2)};
    for (const Range& r : ins)
        if (overlaps(r, ro) || overlaps(r, rl) || overlaps(r, rw))
            return fail(ATTNQAT_E_INVALID, "an output or the workspace overlaps an input");
    if (overlaps(ro, rl) || overlaps(ro, rw) || overlaps(rl, rw))
        return fail(ATTNQAT_E_INVALID, "outputs overlap each other or the workspace");
    if ((rc = check_device())) return rc;

    char* ws = (char*)workspace;
    aq::MxArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.qsb = pl.q.b, a.qsh = pl.q.h, a.qsn = pl.q.n;
    a.ksb = pl.k.b, a.ksh = pl.k.h, a.ksn = pl.k.n;
    a.vsb = pl.v.b, a.vsh = pl.v.h, a.vsn = pl.v.n;
    a.qm = (uint8_t*)(ws + L.qm);
    a.qs = (uint8_t*)(ws + L.qs);
    a.km = (uint8_t*)(ws + L.km);
    a.ks = (uint8_t*)(ws + L.ks);
    a.vtm = (uint8_t*)(ws + L.vtm);
    a.vts = (uint8_t*)(ws + L.vts);
    a.o = (uint16_t*)o;
    a.osb = pl.o.b, a.osh = pl.o.h, a.osn = pl.o.n;
    a.lse = lse;
    a.BH = pl.BH;
    a.H = pl.H;
    a.Nq = (int)pl.Nq;
    a.Nk = (int)pl.Nk;
    a.Nq_pad = (int)pl.Nq_pad;
    a.Nk_pad = (int)pl.Nk_pad;
    a.D = (int)pl.D;
    a.c = p->sm_scale * aq::kLog2e;
    hipStream_t st = (hipStream_t)stream;
    if ((rc = launch(K_MX_QUANT, st, thunk<aq::MxArgs, aq::launch_mx_quant>, &a,
                     "MXFP4 operand quantization")))
        return rc;
    if ((rc = launch(K_MX_FWD, st, thunk<aq::MxArgs, aq::launch_mx_fwd>, &a, "MXFP4 forward")))
        return rc;
    return ok();
}

}  // extern "C"

// C interface of libsdpa (declared in include/sdpa.h): argument checks on the
// host, kernel and launch-shape choice, and launch on the caller's stream.
//
// The argument set mirrors the exactref.ai "scaled_dot_product_attention"
// Arguments table (query, key, value, attn_mask, dropout_p, is_causal, scale,
// enable_gqa); packed variable-length input follows the block-diagonal masks
// of the insureai360 xFormers tutorial, section 4.
#include "sdpa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "api_internal.h"
#include "attn_common.h"

namespace {

thread_local char g_err[512] = "";

sdpa_status fail(sdpa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

sdpa_status ok() {
    g_err[0] = '\0';
    return SDPA_OK;
}

int elem_bytes(sdpa_dtype t) {
    switch (t) {
        case SDPA_F32: return 4;
        case SDPA_F16: return 2;
        case SDPA_BF16: return 2;
        case SDPA_BOOL: return 1;
    }
    return 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks that a tensor can be read with 16-byte vector loads along its rows:
// unit last stride, 16-byte aligned base, and every outer stride (of a dim
// with more than one element) a multiple of 16 bytes.
sdpa_status check_vector_layout(const sdpa_tensor4& t, int ebytes, const char* name) {
    if (t.size[3] == 0) return SDPA_OK;  // zero-width rows: nothing is read or written
    const int64_t vec = 16 / ebytes;
    if (t.size[3] > 1 && t.stride[3] != 1)
        return fail(SDPA_ERR_UNSUPPORTED, "%s: the last dimension must have stride 1", name);
    if (!aligned16(t.data))
        return fail(SDPA_ERR_UNSUPPORTED, "%s: the base pointer must be 16-byte aligned", name);
    for (int d = 0; d < 3; ++d)
        if (t.size[d] > 1 && t.stride[d] % vec != 0)
            return fail(SDPA_ERR_UNSUPPORTED, "%s: stride[%d]=%lld is not a multiple of %lld elements",
                        name, d, (long long)t.stride[d], (long long)vec);
    return SDPA_OK;
}

bool supported_head_dim(int64_t e) { return e == 64 || e == 96 || e == 128; }
// Head dims the forward kernels take: E and Ev multiples of 8 up to 128 (E = 0
// included: the scores are empty sums).  E and Ev in {64, 96, 128} run exact
// instances, the others padded ones (zeros past E and Ev).
bool forward_dims(int64_t e, int64_t ev) {
    return e >= 0 && e <= 128 && e % 8 == 0 && ev >= 0 && ev <= 128 && ev % 8 == 0;
}
// The matrix-core backward takes bf16/fp16 with E == Ev in {64, 96, 128}; the
// vector-ALU backward every other supported call (fp32, Ev != E, other dims).
bool matrix_core_backward(sdpa_dtype dtype, int64_t e, int64_t ev) {
    return dtype != SDPA_F32 && e == ev && supported_head_dim(e);
}

struct Plan {
    bool decode = false;
    int n_splits = 0;
    int keys_per_split = 0;
    size_t workspace = 0;
};

// Split-KV decode applies to few query rows per key/value head, no mask, no
// causal flag, 16-bit inputs.  The automatic split count aims for about 2048
// workgroups (several per compute unit) while keeping each split long enough
// that the final merge stays small next to the key/value stream.
sdpa_status make_plan(sdpa_dtype dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t L, int64_t S,
                      int64_t E, int64_t Ev, bool has_mask, bool causal, int num_splits, Plan* plan) {
    const int64_t group = Hkv > 0 ? Hq / Hkv : 1;
    const bool eligible = !has_mask && !causal && (dtype == SDPA_BF16 || dtype == SDPA_F16) &&
                          L * group <= sdpa::kDecodeMaxRows && L > 0 && supported_head_dim(E) &&
                          supported_head_dim(Ev);
    Plan pl;
    if (num_splits == -1) {
        pl.decode = false;
    } else if (num_splits == 0) {
        pl.decode = eligible && S > 0;
    } else if (num_splits >= 1) {
        if (!eligible)
            return fail(SDPA_ERR_UNSUPPORTED,
                        "the split-KV decode kernel needs no mask, no causal flag, bf16/fp16, head dims "
                        "in {64, 96, 128} and L*Hq/Hkv <= %d (got L=%lld, group=%lld)",
                        sdpa::kDecodeMaxRows, (long long)L, (long long)group);
        pl.decode = true;
    } else {
        return fail(SDPA_ERR_INVALID_ARGUMENT, "num_splits must be -1, 0 or positive (got %d)", num_splits);
    }
    if (pl.decode) {
        const int64_t q = sdpa::kDecodeKeyQuantum;
        int64_t splits;
        if (num_splits >= 1) {
            splits = num_splits;
        } else {
            const int64_t units = B * Hkv > 0 ? B * Hkv : 1;
            splits = (2048 + units - 1) / units;
            const int64_t max_by_len = (S + 255) / 256;
            if (splits > max_by_len) splits = max_by_len;
            if (splits < 1) splits = 1;
        }
        int64_t per = (S + splits - 1) / splits;
        per = ((per + q - 1) / q) * q;
        if (per < q) per = q;
        if (per > (int64_t)1 << 30) return fail(SDPA_ERR_UNSUPPORTED, "key length too large");
        splits = S > 0 ? (S + per - 1) / per : 1;
        pl.n_splits = (int)splits;
        pl.keys_per_split = (int)per;
        const int64_t nrow = B * Hq * L * splits;
        pl.workspace = (size_t)(((nrow + 63) / 64) * 64 + nrow * Ev) * sizeof(float) + 256;
    }
    *plan = pl;
    return SDPA_OK;
}

struct Shapes {
    int64_t B, Hq, Hkv, L, S, E, Ev;
};

sdpa_status check_shapes(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k,
                         const sdpa_tensor4* v, const sdpa_tensor4* attn_mask, int enable_gqa,
                         Shapes* sh) {
    if (dtype != SDPA_F32 && dtype != SDPA_F16 && dtype != SDPA_BF16)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "dtype must be SDPA_F32, SDPA_F16 or SDPA_BF16");
    if (!q || !k || !v) return fail(SDPA_ERR_INVALID_ARGUMENT, "q, k and v descriptors must not be NULL");
    for (int d = 0; d < 4; ++d)
        if (q->size[d] < 0 || k->size[d] < 0 || v->size[d] < 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    Shapes s{q->size[0], q->size[1], k->size[1], q->size[2], k->size[2], q->size[3], v->size[3]};
    if (k->size[0] != s.B || v->size[0] != s.B)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "q, k and v must have the same batch size");
    if (k->size[3] != s.E)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "query and key must share the last dimension E (%lld vs %lld)",
                    (long long)s.E, (long long)k->size[3]);
    if (v->size[2] != s.S || v->size[1] != s.Hkv)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "key and value must share heads and sequence length");
    if (s.Hq != s.Hkv) {
        if (!enable_gqa)
            return fail(SDPA_ERR_INVALID_ARGUMENT,
                        "query has %lld heads and key/value %lld: pass enable_gqa", (long long)s.Hq,
                        (long long)s.Hkv);
        if (s.Hkv == 0 || s.Hq % s.Hkv != 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query heads (%lld) must be a multiple of key/value heads (%lld)",
                        (long long)s.Hq, (long long)s.Hkv);
    }
    if (attn_mask) {
        const int64_t want[4] = {s.B, s.Hq, s.L, s.S};
        for (int d = 0; d < 4; ++d)
            if (attn_mask->size[d] != want[d] && !(attn_mask->size[d] == 1 && d < 3))
                return fail(SDPA_ERR_INVALID_ARGUMENT,
                            "attn_mask size[%d]=%lld does not broadcast to %lld", d,
                            (long long)attn_mask->size[d], (long long)want[d]);
    }
    if (s.L > INT32_MAX || s.S > INT32_MAX || s.Hq > INT32_MAX || s.B > INT32_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "a size exceeds the 32-bit index range of the kernels");
    *sh = s;
    return SDPA_OK;
}

sdpa_status resolve_scale(const double* scale, int64_t E, double* out) {
    if (E == 0) {  // the scores are empty sums (0) and the logits the mask alone: no scale applies
        *out = 1.0;
        return SDPA_OK;
    }
    const double s = scale ? *scale : 1.0 / std::sqrt((double)E);
    if (!std::isfinite(s)) return fail(SDPA_ERR_INVALID_ARGUMENT, "scale must be finite");
    *out = s;
    return SDPA_OK;
}

void fill_scale(sdpa::AttnParams& p, double s) {
    p.neg = s < 0;
    p.scale = (float)s;
    p.scale_abs = (float)std::fabs(s);
    p.scale_log2 = (float)(std::fabs(s) * 1.4426950408889634);
}

hipError_t launch_single_pass(sdpa_dtype dtype, const sdpa::AttnParams& p, int D, bool causal,
                              int mask, bool varlen, hipStream_t s) {
    switch (dtype) {
        case SDPA_BF16: return sdpa::launch_prefill_bf16(p, D, causal, mask, varlen, s);
        case SDPA_F16: return sdpa::launch_prefill_f16(p, D, causal, mask, varlen, s);
        case SDPA_F32: return sdpa::launch_prefill_f32(p, D, causal, mask, varlen, s);
        default: return hipErrorInvalidValue;
    }
}

size_t bwd_workspace_bytes(const Shapes& s) { return (size_t)(s.B * s.Hq * s.L) * sizeof(float) + 256; }

// The dS^T buffer of the backward schedule that stores dS (batched
// matrix-core calls): 16-bit (b, h, key, query), rows padded to a multiple of
// 128 queries.  0 when that schedule does not apply (vector-ALU calls, no
// rows or keys, or more than kBwdDsMaxBytes).
constexpr double kBwdDsMaxBytes = 2.0 * 1024 * 1024 * 1024;
int64_t bwd_ds_row(const Shapes& s) { return (s.L + 127) / 128 * 128; }
size_t bwd_ds_bytes(sdpa_dtype dtype, const Shapes& s) {
    if (!matrix_core_backward(dtype, s.E, s.Ev)) return 0;
    const double bytes = (double)s.B * (double)s.Hq * (double)s.S * (double)bwd_ds_row(s) * 2.0;
    if (bytes <= 0 || bytes > kBwdDsMaxBytes) return 0;
    return (size_t)bytes;
}
// D values (aligned to 256 bytes), then the dS^T buffer (256-byte aligned)
size_t bwd_ds_offset(const Shapes& s) { return ((size_t)(s.B * s.Hq * s.L) * sizeof(float) + 255) / 256 * 256; }
size_t bwd_full_workspace_bytes(sdpa_dtype dtype, const Shapes& s) {
    const size_t ds = bwd_ds_bytes(dtype, s);
    return ds ? 256 + bwd_ds_offset(s) + ds : bwd_workspace_bytes(s);
}

// Shapes and launch plan of a paged-cache call (host only).
struct PagedPlan {
    int64_t B, Hq, Hkv, L, E, Ev, n_pages, page_size;
    int page_shift;
    Plan plan;
};

sdpa_status paged_plan(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* kc,
                       const sdpa_tensor4* vc, int32_t max_seq_len, int enable_gqa, int num_splits,
                       PagedPlan* out) {
    if (dtype != SDPA_BF16 && dtype != SDPA_F16)
        return fail(SDPA_ERR_UNSUPPORTED, "the paged-cache kernel takes bf16 or fp16");
    if (!q || !kc || !vc) return fail(SDPA_ERR_INVALID_ARGUMENT, "q, k_cache and v_cache must not be NULL");
    for (int d = 0; d < 4; ++d)
        if (q->size[d] < 0 || kc->size[d] < 0 || vc->size[d] < 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    PagedPlan pp;
    pp.B = q->size[0]; pp.Hq = q->size[1]; pp.L = q->size[2]; pp.E = q->size[3];
    pp.n_pages = kc->size[0]; pp.Hkv = kc->size[1]; pp.page_size = kc->size[2]; pp.Ev = vc->size[3];
    if (kc->size[3] != pp.E) return fail(SDPA_ERR_INVALID_ARGUMENT, "q and k_cache must share E");
    if (vc->size[0] != pp.n_pages || vc->size[1] != pp.Hkv || vc->size[2] != pp.page_size)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "k_cache and v_cache must share pages, heads and page size");
    if (pp.Hq != pp.Hkv) {
        if (!enable_gqa)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query has %lld heads and the cache %lld: pass enable_gqa",
                        (long long)pp.Hq, (long long)pp.Hkv);
        if (pp.Hkv == 0 || pp.Hq % pp.Hkv != 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query heads must be a multiple of cache heads");
    }
    if (max_seq_len < 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "max_seq_len must be non-negative");
    int shift = 0;
    while (shift < 30 && ((int64_t)1 << shift) < pp.page_size) ++shift;
    if (pp.page_size < 16 || ((int64_t)1 << shift) != pp.page_size)
        return fail(SDPA_ERR_UNSUPPORTED, "page_size must be a power of two >= 16 (got %lld)",
                    (long long)pp.page_size);
    pp.page_shift = shift;
    const int64_t group = pp.Hkv > 0 ? pp.Hq / pp.Hkv : 1;
    if (!forward_dims(pp.E, pp.Ev))
        return fail(SDPA_ERR_UNSUPPORTED, "head dims E=%lld, Ev=%lld: each must be a multiple of 8 up to 128",
                    (long long)pp.E, (long long)pp.Ev);
    if (num_splits < 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "num_splits must be 0 or positive");
    // the split-KV decode kernel takes head dims in {64, 96, 128}; other dims always
    // run the single-pass kernel, decode steps included
    const bool exact = supported_head_dim(pp.E) && supported_head_dim(pp.Ev);
    if (!exact && num_splits > 0)
        return fail(SDPA_ERR_UNSUPPORTED, "split-KV needs head dims in {64, 96, 128} (got E=%lld, Ev=%lld)",
                    (long long)pp.E, (long long)pp.Ev);
    if (pp.L * group > sdpa::kDecodeMaxRows || !exact) {
        // chunked prefill: the single-pass kernel reads the pages itself, no workspace
        if (num_splits > 0)
            return fail(SDPA_ERR_UNSUPPORTED,
                        "split-KV needs L * Hq / Hkv <= %d new rows per cache head (got %lld)",
                        sdpa::kDecodeMaxRows, (long long)(pp.L * group));
        pp.plan = Plan();
        *out = pp;
        return SDPA_OK;
    }
    // Splits as for the dense split-KV path (about 2048 workgroups), each a
    // multiple of 128 keys spanning at most 64 pages (a split's pages sit in
    // the 64 lanes of a wavefront).  At least one split, so that rows with no cached
    // key still get output 0 and lse -inf from the merge.
    const int64_t quantum = sdpa::kDecodeKeyQuantum;
    const int64_t S = max_seq_len;
    int64_t splits = num_splits;
    if (splits == 0) {
        const int64_t units = pp.B * pp.Hkv > 0 ? pp.B * pp.Hkv : 1;
        splits = (2048 + units - 1) / units;
        const int64_t max_by_len = (S + 255) / 256;
        if (splits > max_by_len) splits = max_by_len;
        if (splits < 1) splits = 1;
    }
    int64_t per = S > 0 ? (S + splits - 1) / splits : quantum;
    per = ((per + quantum - 1) / quantum) * quantum;
    // 63 pages of keys: a split that starts inside a page then spans at most 64
    const int64_t cap = (63 * pp.page_size / quantum) * quantum;
    if (per > cap) per = cap;
    if (per < quantum) per = quantum;
    Plan pl;
    pl.decode = true;
    pl.n_splits = (int)(S > 0 ? (S + per - 1) / per : 1);
    pl.keys_per_split = (int)per;
    const int64_t nrow = pp.B * pp.Hq * pp.L * pl.n_splits;
    pl.workspace = (size_t)(((nrow + 63) / 64) * 64 + nrow * pp.Ev) * sizeof(float) + 256;
    pp.plan = pl;
    *out = pp;
    return SDPA_OK;
}

}  // namespace

namespace sdpa {
sdpa_status record_error(sdpa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace sdpa

extern "C" {

int sdpa_abi_version(void) { return 5; }

const char* sdpa_last_error(void) { return g_err; }

sdpa_status sdpa_fwd_workspace_size(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k,
                                    const sdpa_tensor4* v, const sdpa_tensor4* attn_mask,
                                    int is_causal, int enable_gqa, int num_splits, size_t* bytes) {
    if (!bytes) return fail(SDPA_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
    Shapes s;
    sdpa_status st = check_shapes(dtype, q, k, v, attn_mask, enable_gqa, &s);
    if (st != SDPA_OK) return st;
    Plan pl;
    st = make_plan(dtype, s.B, s.Hq, s.Hkv, s.L, s.S, s.E, s.Ev, attn_mask != nullptr, is_causal != 0,
                   num_splits, &pl);
    if (st != SDPA_OK) return st;
    *bytes = pl.workspace;
    return ok();
}

sdpa_status sdpa_fwd(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k,
                     const sdpa_tensor4* v, const sdpa_tensor4* attn_mask, sdpa_dtype mask_dtype,
                     double dropout_p, int is_causal, const double* scale, int enable_gqa,
                     const sdpa_tensor4* out, const sdpa_tensor4* lse, void* workspace,
                     size_t workspace_bytes, int num_splits, void* stream) {
    if (dropout_p != 0.0)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "dropout_p must be 0: a random dropout has no exact reference");
    Shapes s;
    sdpa_status st = check_shapes(dtype, q, k, v, attn_mask, enable_gqa, &s);
    if (st != SDPA_OK) return st;
    if (!out || !lse) return fail(SDPA_ERR_INVALID_ARGUMENT, "out and lse descriptors must not be NULL");
    const int64_t want_o[4] = {s.B, s.Hq, s.L, s.Ev};
    for (int d = 0; d < 4; ++d) {
        if (out->size[d] != want_o[d])
            return fail(SDPA_ERR_INVALID_ARGUMENT, "out must be (B, Hq, L, Ev)");
        if (d < 3 && lse->size[d] != want_o[d])
            return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must be (B, Hq, L, 1)");
    }
    if (lse->size[3] != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must be (B, Hq, L, 1)");
    if (attn_mask && mask_dtype != SDPA_F32 && mask_dtype != SDPA_BOOL)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_mask must be SDPA_F32 (added) or SDPA_BOOL (keep)");
    if (s.B * s.Hq * s.L == 0) return ok();  // nothing to compute
    if (!forward_dims(s.E, s.Ev))
        return fail(SDPA_ERR_UNSUPPORTED, "head dims E=%lld, Ev=%lld: each must be a multiple of 8 up to 128",
                    (long long)s.E, (long long)s.Ev);
    const int eb = elem_bytes(dtype);
    if ((st = check_vector_layout(*q, eb, "q")) != SDPA_OK) return st;
    if (s.S > 0) {
        if ((st = check_vector_layout(*k, eb, "k")) != SDPA_OK) return st;
        if ((st = check_vector_layout(*v, eb, "v")) != SDPA_OK) return st;
    }
    if ((st = check_vector_layout(*out, eb, "out")) != SDPA_OK) return st;
    if (!lse->data) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse data must not be NULL");
    if (attn_mask) {
        if (!attn_mask->data && s.S > 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_mask data is NULL");
        if (s.S > 1 && attn_mask->stride[3] != 1)
            return fail(SDPA_ERR_UNSUPPORTED, "attn_mask: the key dimension must have stride 1");
    }
    double sc;
    if ((st = resolve_scale(scale, s.E, &sc)) != SDPA_OK) return st;
    Plan pl;
    if ((st = make_plan(dtype, s.B, s.Hq, s.Hkv, s.L, s.S, s.E, s.Ev, attn_mask != nullptr, is_causal != 0,
                        num_splits, &pl)) != SDPA_OK)
        return st;
    if (pl.workspace > workspace_bytes || (pl.workspace > 0 && !workspace))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes needed, %zu given",
                    pl.workspace, workspace_bytes);
    hipStream_t hs = (hipStream_t)stream;
    const int64_t lse_sb = lse->size[0] > 1 ? lse->stride[0] : 0;
    const int64_t lse_sh = lse->size[1] > 1 ? lse->stride[1] : 0;
    const int64_t lse_sr = lse->size[2] > 1 ? lse->stride[2] : 1;
    if (lse_sr != 1) return fail(SDPA_ERR_UNSUPPORTED, "lse: the query dimension must have stride 1");

    if (pl.decode) {
        sdpa::DecodeParams p{};
        p.q = q->data; p.k = k->data; p.v = v->data; p.o = out->data; p.lse = (float*)lse->data;
        float* ws = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
        p.part_lse = ws;
        const int64_t nrow = s.B * s.Hq * s.L * pl.n_splits;
        p.part_o = ws + ((nrow + 63) / 64) * 64;
        p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_sr = q->stride[2];
        p.k_sb = k->stride[0]; p.k_sh = k->stride[1]; p.k_sr = k->stride[2];
        p.v_sb = v->stride[0]; p.v_sh = v->stride[1]; p.v_sr = v->stride[2];
        p.o_sb = out->stride[0]; p.o_sh = out->stride[1]; p.o_sr = out->stride[2];
        p.lse_sb = lse_sb; p.lse_sh = lse_sh;
        p.B = (int)s.B; p.Hq = (int)s.Hq; p.Hkv = (int)s.Hkv; p.group = (int)(s.Hq / s.Hkv);
        p.L = (int)s.L; p.S = (int)s.S;
        p.rows = (int)(s.L * p.group);
        p.dv = (int)s.Ev;
        p.n_splits = pl.n_splits;
        p.keys_per_split = pl.keys_per_split;
        p.neg = sc < 0;
        p.scale_log2 = (float)(std::fabs(sc) * 1.4426950408889634);
        hipError_t e = sdpa::launch_decode(p, dtype == SDPA_BF16 ? sdpa::ELEM_BF16 : sdpa::ELEM_F16,
                                           (int)s.E, hs);
        if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
        return ok();
    }

    sdpa::AttnParams p{};
    p.q = q->data; p.k = k->data; p.v = v->data; p.o = out->data; p.lse = (float*)lse->data;
    p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_sr = q->stride[2];
    p.k_sb = k->stride[0]; p.k_sh = k->stride[1]; p.k_sr = k->stride[2];
    p.v_sb = v->stride[0]; p.v_sh = v->stride[1]; p.v_sr = v->stride[2];
    p.o_sb = out->stride[0]; p.o_sh = out->stride[1]; p.o_sr = out->stride[2];
    p.lse_sb = lse_sb; p.lse_sh = lse_sh;
    int mask_kind = sdpa::MASK_NONE;
    if (attn_mask) {
        mask_kind = mask_dtype == SDPA_F32 ? sdpa::MASK_FLOAT : sdpa::MASK_BOOL;
        p.mask = attn_mask->data;
        p.m_sb = attn_mask->size[0] > 1 ? attn_mask->stride[0] : 0;
        p.m_sh = attn_mask->size[1] > 1 ? attn_mask->stride[1] : 0;
        p.m_sr = attn_mask->size[2] > 1 ? attn_mask->stride[2] : 0;
        const int64_t mvec = mask_dtype == SDPA_F32 ? 4 : 8;  // elements per vector load
        const int64_t mal = mask_dtype == SDPA_F32 ? 16 : 8;  // its alignment in bytes
        // vector loads also need whole vectors at the end of each row
        p.mask_vec = ((uintptr_t)attn_mask->data % mal == 0) && p.m_sb % mvec == 0 &&
                     p.m_sh % mvec == 0 && p.m_sr % mvec == 0 && s.S % mvec == 0;
        // bit 1 (bool masks): rows in whole 16-byte chunks, for the eight-wave kernel
        if (mask_dtype == SDPA_BOOL && (uintptr_t)attn_mask->data % 16 == 0 && p.m_sb % 16 == 0 &&
            p.m_sh % 16 == 0 && p.m_sr % 16 == 0 && s.S % 16 == 0)
            p.mask_vec |= 2;
    }
    p.B = (int)s.B; p.Hq = (int)s.Hq; p.Hkv = (int)s.Hkv; p.group = (int)(s.Hq / s.Hkv);
    p.L = (int)s.L; p.S = (int)s.S;
    p.dv = (int)s.Ev;
    p.e = (int)s.E;
    const int bm = dtype == SDPA_F32 ? sdpa::kF32BlockM : sdpa::kPrefillBlockM;
    p.n_qtiles = (int)((s.L + bm - 1) / bm);
    fill_scale(p, sc);
    hipError_t e = launch_single_pass(dtype, p, (int)s.E, is_causal != 0, mask_kind, false, hs);
    if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

sdpa_status sdpa_fwd_varlen(sdpa_dtype dtype, const void* q, int64_t q_stride_tok,
                            int64_t q_stride_head, const void* k, int64_t k_stride_tok,
                            int64_t k_stride_head, const void* v, int64_t v_stride_tok,
                            int64_t v_stride_head, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t n_seqs, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t E, int32_t Ev,
                            int64_t total_q, int64_t total_k, double dropout_p, int is_causal,
                            const double* scale, int enable_gqa, void* out, int64_t o_stride_tok,
                            int64_t o_stride_head, float* lse, int64_t lse_stride_head,
                            void* stream) {
    if (dropout_p != 0.0)
        return fail(SDPA_ERR_INVALID_ARGUMENT,
                    "dropout_p must be 0: a random dropout has no exact reference");
    if (dtype != SDPA_F32 && dtype != SDPA_F16 && dtype != SDPA_BF16)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "dtype must be SDPA_F32, SDPA_F16 or SDPA_BF16");
    if (n_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || Hq < 0 || Hkv < 0 || E < 0 || Ev < 0 ||
        total_q < 0 || total_k < 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    if (Hq != Hkv) {
        if (!enable_gqa)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query has %d heads and key/value %d: pass enable_gqa",
                        Hq, Hkv);
        if (Hkv == 0 || Hq % Hkv != 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query heads (%d) must be a multiple of key/value heads (%d)",
                        Hq, Hkv);
    }
    if (n_seqs == 0 || max_seqlen_q == 0 || Hq == 0 || total_q == 0) return ok();
    if (!cu_seqlens_q || !cu_seqlens_k)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must not be NULL");
    if (!forward_dims(E, Ev))
        return fail(SDPA_ERR_UNSUPPORTED, "head dims E=%d, Ev=%d: each must be a multiple of 8 up to 128", E, Ev);
    // (zero-width rows are never touched, so their tensors may be empty and NULL)
    if ((E > 0 && !q) || (Ev > 0 && !out) || !lse || (total_k > 0 && ((E > 0 && !k) || (Ev > 0 && !v))))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "data pointers must not be NULL");
    const int64_t vec = 16 / elem_bytes(dtype);
    const void* ptrs[4] = {q, k, v, out};
    const int64_t strides[8] = {q_stride_tok, q_stride_head, k_stride_tok, k_stride_head,
                                v_stride_tok, v_stride_head, o_stride_tok, o_stride_head};
    const bool used[4] = {E > 0, E > 0, Ev > 0, Ev > 0};  // zero-width rows are never read or written
    for (int i = 0; i < 4; ++i)
        if (used[i] && ptrs[i] && !aligned16(ptrs[i]))
            return fail(SDPA_ERR_UNSUPPORTED, "packed tensors need 16-byte aligned base pointers");
    for (int i = 0; i < 8; ++i)
        if (used[i / 2] && strides[i] % vec != 0)
            return fail(SDPA_ERR_UNSUPPORTED, "packed strides must be multiples of %lld elements", (long long)vec);
    double sc;
    sdpa_status st;
    if ((st = resolve_scale(scale, E, &sc)) != SDPA_OK) return st;
    sdpa::AttnParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
    p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
    p.q_sr = q_stride_tok; p.q_sh = q_stride_head;
    p.k_sr = k_stride_tok; p.k_sh = k_stride_head;
    p.v_sr = v_stride_tok; p.v_sh = v_stride_head;
    p.o_sr = o_stride_tok; p.o_sh = o_stride_head;
    p.lse_sh = lse_stride_head;
    p.total_q = total_q; p.total_k = total_k;
    p.B = n_seqs; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
    p.L = max_seqlen_q; p.S = max_seqlen_k;
    p.dv = Ev;
    p.e = E;
    const int bm = dtype == SDPA_F32 ? sdpa::kF32BlockM : sdpa::kPrefillBlockM;
    p.n_qtiles = (max_seqlen_q + bm - 1) / bm;
    fill_scale(p, sc);
    hipError_t e = launch_single_pass(dtype, p, E, is_causal != 0, sdpa::MASK_NONE, true,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "launch failed: %s", hipGetErrorString(e));
    return ok();
}

sdpa_status sdpa_fwd_paged_workspace_size(sdpa_dtype dtype, const sdpa_tensor4* q,
                                          const sdpa_tensor4* k_cache, const sdpa_tensor4* v_cache,
                                          int32_t max_seq_len, int enable_gqa, int num_splits,
                                          size_t* bytes) {
    if (!bytes) return fail(SDPA_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
    PagedPlan pp;
    sdpa_status st = paged_plan(dtype, q, k_cache, v_cache, max_seq_len, enable_gqa, num_splits, &pp);
    if (st != SDPA_OK) return st;
    *bytes = pp.plan.workspace;
    return ok();
}

sdpa_status sdpa_fwd_paged(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k_cache,
                           const sdpa_tensor4* v_cache, const int32_t* block_table, int64_t bt_stride,
                           int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                           int is_causal, const double* scale, int enable_gqa,
                           const sdpa_tensor4* out, const sdpa_tensor4* lse, void* workspace,
                           size_t workspace_bytes, int num_splits, void* stream) {
    PagedPlan pp;
    sdpa_status st = paged_plan(dtype, q, k_cache, v_cache, max_seq_len, enable_gqa, num_splits, &pp);
    if (st != SDPA_OK) return st;
    if (!out || !lse) return fail(SDPA_ERR_INVALID_ARGUMENT, "out and lse descriptors must not be NULL");
    const int64_t want_o[4] = {pp.B, pp.Hq, pp.L, pp.Ev};
    for (int d = 0; d < 4; ++d) {
        if (out->size[d] != want_o[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "out must be (B, Hq, L, Ev)");
        if (d < 3 && lse->size[d] != want_o[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must be (B, Hq, L, 1)");
    }
    if (lse->size[3] != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must be (B, Hq, L, 1)");
    if (pp.B * pp.Hq * pp.L == 0) return ok();
    if (max_blocks < 0 || bt_stride < max_blocks)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "need 0 <= max_blocks <= bt_stride");
    if (!block_table || !seq_lens) return fail(SDPA_ERR_INVALID_ARGUMENT, "block_table and seq_lens must not be NULL");
    if ((int64_t)max_blocks * pp.page_size > INT32_MAX || pp.n_pages > INT32_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "cache too large for 32-bit key indices");
    const int eb = elem_bytes(dtype);
    if ((st = check_vector_layout(*q, eb, "q")) != SDPA_OK) return st;
    if (pp.n_pages > 0) {
        if ((st = check_vector_layout(*k_cache, eb, "k_cache")) != SDPA_OK) return st;
        if ((st = check_vector_layout(*v_cache, eb, "v_cache")) != SDPA_OK) return st;
    }
    if ((st = check_vector_layout(*out, eb, "out")) != SDPA_OK) return st;
    if (!lse->data) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse data must not be NULL");
    const int64_t lse_sr = lse->size[2] > 1 ? lse->stride[2] : 1;
    if (lse_sr != 1) return fail(SDPA_ERR_UNSUPPORTED, "lse: the query dimension must have stride 1");
    double sc;
    if ((st = resolve_scale(scale, pp.E, &sc)) != SDPA_OK) return st;
    if (pp.plan.workspace > workspace_bytes || (pp.plan.workspace > 0 && !workspace))
        return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes needed, %zu given",
                    pp.plan.workspace, workspace_bytes);
    if (!pp.plan.decode) {
        sdpa::AttnParams a{};
        a.q = q->data; a.k = k_cache->data; a.v = v_cache->data; a.o = out->data; a.lse = (float*)lse->data;
        a.q_sb = q->stride[0]; a.q_sh = q->stride[1]; a.q_sr = q->stride[2];
        a.k_sb = k_cache->stride[0]; a.k_sh = k_cache->stride[1]; a.k_sr = k_cache->stride[2];
        a.v_sb = v_cache->stride[0]; a.v_sh = v_cache->stride[1]; a.v_sr = v_cache->stride[2];
        a.o_sb = out->stride[0]; a.o_sh = out->stride[1]; a.o_sr = out->stride[2];
        a.lse_sb = lse->size[0] > 1 ? lse->stride[0] : 0;
        a.lse_sh = lse->size[1] > 1 ? lse->stride[1] : 0;
        a.B = (int)pp.B; a.Hq = (int)pp.Hq; a.Hkv = (int)pp.Hkv; a.group = (int)(pp.Hq / pp.Hkv);
        a.L = (int)pp.L; a.S = max_seq_len;
        a.dv = (int)pp.Ev;
        a.e = (int)pp.E;
        a.n_qtiles = (int)((pp.L + sdpa::kPrefillBlockM - 1) / sdpa::kPrefillBlockM);
        fill_scale(a, sc);
        a.block_table = block_table;
        a.seq_lens = seq_lens;
        a.bt_stride = bt_stride;
        a.page_shift = pp.page_shift;
        a.n_pages = (int)pp.n_pages;
        a.max_blocks = max_blocks;
        hipError_t e = launch_single_pass(dtype, a, (int)pp.E, is_causal != 0, sdpa::MASK_NONE, false,
                                          (hipStream_t)stream);
        if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "paged prefill launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    sdpa::DecodeParams p{};
    p.q = q->data; p.k = k_cache->data; p.v = v_cache->data; p.o = out->data; p.lse = (float*)lse->data;
    float* ws = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    p.part_lse = ws;
    const int64_t nrow = pp.B * pp.Hq * pp.L * pp.plan.n_splits;
    p.part_o = ws + ((nrow + 63) / 64) * 64;
    p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_sr = q->stride[2];
    p.k_sb = k_cache->stride[0]; p.k_sh = k_cache->stride[1]; p.k_sr = k_cache->stride[2];
    p.v_sb = v_cache->stride[0]; p.v_sh = v_cache->stride[1]; p.v_sr = v_cache->stride[2];
    p.o_sb = out->stride[0]; p.o_sh = out->stride[1]; p.o_sr = out->stride[2];
    p.lse_sb = lse->size[0] > 1 ? lse->stride[0] : 0;
    p.lse_sh = lse->size[1] > 1 ? lse->stride[1] : 0;
    p.B = (int)pp.B; p.Hq = (int)pp.Hq; p.Hkv = (int)pp.Hkv; p.group = (int)(pp.Hq / pp.Hkv);
    p.L = (int)pp.L; p.S = max_seq_len;
    p.rows = (int)(pp.L * p.group);
    p.dv = (int)pp.Ev;
    p.n_splits = pp.plan.n_splits;
    p.keys_per_split = pp.plan.keys_per_split;
    p.neg = sc < 0;
    p.scale_log2 = (float)(std::fabs(sc) * 1.4426950408889634);
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.bt_stride = bt_stride;
    p.page_shift = pp.page_shift;
    p.n_pages = (int)pp.n_pages;
    p.max_blocks = max_blocks;
    p.causal = is_causal != 0;
    hipError_t e = sdpa::launch_decode(p, dtype == SDPA_BF16 ? sdpa::ELEM_BF16 : sdpa::ELEM_F16, (int)pp.E,
                                       (hipStream_t)stream);
    if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "paged decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

sdpa_status sdpa_fwd_paged_varlen(sdpa_dtype dtype, const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                                  const int32_t* cu_seqlens_q, int32_t n_seqs, int32_t max_seqlen_q,
                                  int64_t total_q, int32_t Hq, const sdpa_tensor4* k_cache,
                                  const sdpa_tensor4* v_cache, const int32_t* block_table, int64_t bt_stride,
                                  int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                                  int is_causal, const double* scale, int enable_gqa, void* out,
                                  int64_t o_stride_tok, int64_t o_stride_head, float* lse,
                                  int64_t lse_stride_head, void* stream) {
    if (dtype != SDPA_BF16 && dtype != SDPA_F16)
        return fail(dtype == SDPA_F32 ? SDPA_ERR_UNSUPPORTED : SDPA_ERR_INVALID_ARGUMENT,
                    "the paged-cache kernels take bf16 or fp16");
    if (!k_cache || !v_cache) return fail(SDPA_ERR_INVALID_ARGUMENT, "k_cache and v_cache must not be NULL");
    for (int d = 0; d < 4; ++d)
        if (k_cache->size[d] < 0 || v_cache->size[d] < 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    if (n_seqs < 0 || max_seqlen_q < 0 || total_q < 0 || Hq < 0 || max_seq_len < 0 || max_blocks < 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    const int64_t n_pages = k_cache->size[0], Hkv = k_cache->size[1], ps = k_cache->size[2];
    const int64_t E = k_cache->size[3], Ev = v_cache->size[3];
    if (v_cache->size[0] != n_pages || v_cache->size[1] != Hkv || v_cache->size[2] != ps)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "k_cache and v_cache must share pages, heads and page size");
    if (Hq != Hkv) {
        if (!enable_gqa)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query has %d heads and the cache %lld: pass enable_gqa", Hq,
                        (long long)Hkv);
        if (Hkv == 0 || Hq % Hkv != 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query heads must be a multiple of cache heads");
    }
    int shift = 0;
    while (shift < 30 && ((int64_t)1 << shift) < ps) ++shift;
    if (ps < 16 || ((int64_t)1 << shift) != ps)
        return fail(SDPA_ERR_UNSUPPORTED, "page_size must be a power of two >= 16 (got %lld)", (long long)ps);
    if (!forward_dims(E, Ev))
        return fail(SDPA_ERR_UNSUPPORTED, "head dims E=%lld, Ev=%lld: each must be a multiple of 8 up to 128",
                    (long long)E, (long long)Ev);
    if (bt_stride < max_blocks) return fail(SDPA_ERR_INVALID_ARGUMENT, "need 0 <= max_blocks <= bt_stride");
    if ((int64_t)max_blocks * ps > INT32_MAX || n_pages > INT32_MAX)
        return fail(SDPA_ERR_UNSUPPORTED, "cache too large for 32-bit key indices");
    if (n_seqs == 0 || total_q == 0 || Hq == 0 || max_seqlen_q == 0) return ok();
    if (!cu_seqlens_q || !block_table || !seq_lens)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "cu_seqlens_q, block_table and seq_lens must not be NULL");
    if ((E > 0 && !q) || (Ev > 0 && !out) || !lse)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "data pointers must not be NULL");
    const int eb = elem_bytes(dtype);
    const int64_t vec = 16 / eb;
    if ((E > 0 && !aligned16(q)) || (Ev > 0 && !aligned16(out)))
        return fail(SDPA_ERR_UNSUPPORTED, "packed tensors need 16-byte aligned base pointers");
    const int64_t strides[4] = {q_stride_tok, q_stride_head, o_stride_tok, o_stride_head};
    for (int i = 0; i < 4; ++i)
        if ((i < 2 ? E : Ev) > 0 && strides[i] % vec != 0)
            return fail(SDPA_ERR_UNSUPPORTED, "packed strides must be multiples of %lld elements", (long long)vec);
    sdpa_status st;
    if (n_pages > 0) {
        if ((st = check_vector_layout(*k_cache, eb, "k_cache")) != SDPA_OK) return st;
        if ((st = check_vector_layout(*v_cache, eb, "v_cache")) != SDPA_OK) return st;
    }
    double sc;
    if ((st = resolve_scale(scale, E, &sc)) != SDPA_OK) return st;
    sdpa::AttnParams a{};
    a.q = q; a.k = k_cache->data; a.v = v_cache->data; a.o = out; a.lse = lse;
    a.cu_q = cu_seqlens_q;
    a.q_sr = q_stride_tok; a.q_sh = q_stride_head;
    a.k_sb = k_cache->stride[0]; a.k_sh = k_cache->stride[1]; a.k_sr = k_cache->stride[2];
    a.v_sb = v_cache->stride[0]; a.v_sh = v_cache->stride[1]; a.v_sr = v_cache->stride[2];
    a.o_sr = o_stride_tok; a.o_sh = o_stride_head;
    a.lse_sh = lse_stride_head;
    a.total_q = total_q;
    a.B = n_seqs; a.Hq = Hq; a.Hkv = (int)Hkv; a.group = (int)(Hq / Hkv);
    a.L = max_seqlen_q; a.S = max_seq_len;
    a.dv = (int)Ev; a.e = (int)E;
    a.n_qtiles = (max_seqlen_q + sdpa::kPrefillBlockM - 1) / sdpa::kPrefillBlockM;
    fill_scale(a, sc);
    a.block_table = block_table; a.seq_lens = seq_lens; a.bt_stride = bt_stride;
    a.page_shift = shift; a.n_pages = (int)n_pages; a.max_blocks = max_blocks;
    hipError_t e = launch_single_pass(dtype, a, (int)E, is_causal != 0, sdpa::MASK_NONE, true, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "paged prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

sdpa_status sdpa_bwd_workspace_size(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k,
                                    const sdpa_tensor4* v, int enable_gqa, size_t* bytes) {
    if (!bytes) return fail(SDPA_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
    Shapes s;
    sdpa_status st = check_shapes(dtype, q, k, v, nullptr, enable_gqa, &s);
    if (st != SDPA_OK) return st;
    *bytes = bwd_full_workspace_bytes(dtype, s);
    return ok();
}

sdpa_status sdpa_bwd(sdpa_dtype dtype, const sdpa_tensor4* q, const sdpa_tensor4* k,
                     const sdpa_tensor4* v, const sdpa_tensor4* attn_mask, sdpa_dtype mask_dtype,
                     const sdpa_tensor4* out, const sdpa_tensor4* lse,
                     const sdpa_tensor4* dout, int is_causal, const double* scale, int enable_gqa,
                     const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv,
                     void* workspace, size_t workspace_bytes, void* stream) {
    Shapes s;
    sdpa_status st = check_shapes(dtype, q, k, v, attn_mask, enable_gqa, &s);
    if (st != SDPA_OK) return st;
    if (attn_mask && mask_dtype != SDPA_F32 && mask_dtype != SDPA_BOOL)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_mask must be SDPA_F32 (added) or SDPA_BOOL (keep)");
    if (!out || !lse || !dout || !dq || !dk || !dv)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "out, lse, dout, dq, dk and dv descriptors must not be NULL");
    const int64_t want_o[4] = {s.B, s.Hq, s.L, s.Ev};
    const int64_t want_q[4] = {s.B, s.Hq, s.L, s.E};
    const int64_t want_k[4] = {s.B, s.Hkv, s.S, s.E};
    const int64_t want_v[4] = {s.B, s.Hkv, s.S, s.Ev};
    for (int d = 0; d < 4; ++d) {
        if (out->size[d] != want_o[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "out must be (B, Hq, L, Ev)");
        if (dout->size[d] != want_o[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "dout must be (B, Hq, L, Ev)");
        if (dq->size[d] != want_q[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "dq must be (B, Hq, L, E)");
        if (dk->size[d] != want_k[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "dk must be (B, Hkv, S, E)");
        if (dv->size[d] != want_v[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "dv must be (B, Hkv, S, Ev)");
        if (d < 3 && lse->size[d] != want_o[d]) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must be (B, Hq, L, 1)");
    }
    if (lse->size[3] != 1) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must be (B, Hq, L, 1)");
    if (s.B * s.Hq * s.L == 0 && s.B * s.Hkv * s.S == 0) return ok();  // nothing to compute
    if (!forward_dims(s.E, s.Ev))
        return fail(SDPA_ERR_UNSUPPORTED, "head dims E=%lld, Ev=%lld: each must be a multiple of 8 up to 128",
                    (long long)s.E, (long long)s.Ev);
    const int eb = elem_bytes(dtype);
    const sdpa_tensor4* vec_t[8] = {q, k, v, out, dout, dq, dk, dv};
    const char* vec_n[8] = {"q", "k", "v", "out", "dout", "dq", "dk", "dv"};
    for (int i = 0; i < 8; ++i) {
        const bool empty = vec_t[i]->size[0] * vec_t[i]->size[1] * vec_t[i]->size[2] == 0;
        if (!empty && (st = check_vector_layout(*vec_t[i], eb, vec_n[i])) != SDPA_OK) return st;
    }
    if (s.L > 0 && !lse->data) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse data must not be NULL");
    const int64_t lse_sr = lse->size[2] > 1 ? lse->stride[2] : 1;
    if (lse_sr != 1) return fail(SDPA_ERR_UNSUPPORTED, "lse: the query dimension must have stride 1");
    if (attn_mask) {
        if (!attn_mask->data && s.S > 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "attn_mask data is NULL");
        if (s.S > 1 && attn_mask->stride[3] != 1)
            return fail(SDPA_ERR_UNSUPPORTED, "attn_mask: the key dimension must have stride 1");
    }
    double sc;
    if ((st = resolve_scale(scale, s.E, &sc)) != SDPA_OK) return st;
    const size_t need = bwd_workspace_bytes(s);
    if (workspace_bytes < need || !workspace)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes needed, %zu given", need,
                    workspace_bytes);

    sdpa::BwdParams p{};
    p.q = q->data; p.k = k->data; p.v = v->data; p.o = out->data; p.dout = dout->data;
    p.lse = (const float*)lse->data;
    p.dsum = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    // a workspace of sdpa_bwd_workspace_size bytes also holds dS^T: the
    // schedule with one matrix product for dQ; a smaller one: dQ recomputes
    // S and dP
    if (bwd_ds_bytes(dtype, s) > 0 && workspace_bytes >= bwd_full_workspace_bytes(dtype, s)) {
        p.ds = (uint16_t*)((char*)p.dsum + bwd_ds_offset(s));
        p.ds_lp = bwd_ds_row(s);
    }
    p.dq = dq->data; p.dk = dk->data; p.dv = dv->data;
    p.q_sb = q->stride[0]; p.q_sh = q->stride[1]; p.q_sr = q->stride[2];
    p.k_sb = k->stride[0]; p.k_sh = k->stride[1]; p.k_sr = k->stride[2];
    p.v_sb = v->stride[0]; p.v_sh = v->stride[1]; p.v_sr = v->stride[2];
    p.o_sb = out->stride[0]; p.o_sh = out->stride[1]; p.o_sr = out->stride[2];
    p.do_sb = dout->stride[0]; p.do_sh = dout->stride[1]; p.do_sr = dout->stride[2];
    p.dq_sb = dq->stride[0]; p.dq_sh = dq->stride[1]; p.dq_sr = dq->stride[2];
    p.dk_sb = dk->stride[0]; p.dk_sh = dk->stride[1]; p.dk_sr = dk->stride[2];
    p.dv_sb = dv->stride[0]; p.dv_sh = dv->stride[1]; p.dv_sr = dv->stride[2];
    p.lse_sb = lse->size[0] > 1 ? lse->stride[0] : 0;
    p.lse_sh = lse->size[1] > 1 ? lse->stride[1] : 0;
    p.B = (int)s.B; p.Hq = (int)s.Hq; p.Hkv = (int)s.Hkv; p.group = (int)(s.Hq / s.Hkv);
    p.L = (int)s.L; p.S = (int)s.S;
    p.n_qtiles = (int)((s.L + 127) / 128);
    p.n_ktiles = (int)((s.S + 127) / 128);
    p.elem = dtype == SDPA_BF16 ? sdpa::ELEM_BF16 : dtype == SDPA_F16 ? sdpa::ELEM_F16 : sdpa::ELEM_F32;
    p.scale = (float)sc;
    p.e = (int)s.E; p.ev = (int)s.Ev;
    int mask_kind = sdpa::MASK_NONE;
    if (attn_mask) {
        mask_kind = mask_dtype == SDPA_F32 ? sdpa::MASK_FLOAT : sdpa::MASK_BOOL;
        p.mask = attn_mask->data;
        p.m_sb = attn_mask->size[0] > 1 ? attn_mask->stride[0] : 0;
        p.m_sh = attn_mask->size[1] > 1 ? attn_mask->stride[1] : 0;
        p.m_sr = attn_mask->size[2] > 1 ? attn_mask->stride[2] : 0;
        // vector loads: aligned runs, and whole vectors at the end of each row
        const int64_t mvec = mask_dtype == SDPA_F32 ? 4 : 8, mal = mask_dtype == SDPA_F32 ? 16 : 8;
        p.mask_vec = ((uintptr_t)attn_mask->data % mal == 0) && p.m_sb % mvec == 0 && p.m_sh % mvec == 0 &&
                     p.m_sr % mvec == 0 && s.S % mvec == 0;
    }
    hipError_t e = matrix_core_backward(dtype, s.E, s.Ev)
                       ? sdpa::launch_backward(p, (int)s.E, is_causal != 0, mask_kind, false, (hipStream_t)stream)
                       : sdpa::launch_backward_vec(p, is_causal != 0, mask_kind, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

sdpa_status sdpa_bwd_varlen_workspace_size(int32_t Hq, int64_t total_q, size_t* bytes) {
    if (!bytes) return fail(SDPA_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
    if (Hq < 0 || total_q < 0) return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    *bytes = (size_t)Hq * (size_t)total_q * sizeof(float) + 256;
    return ok();
}

sdpa_status sdpa_bwd_varlen(sdpa_dtype dtype, const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                            const void* k, int64_t k_stride_tok, int64_t k_stride_head, const void* v,
                            int64_t v_stride_tok, int64_t v_stride_head, const void* out, int64_t o_stride_tok,
                            int64_t o_stride_head, const float* lse, int64_t lse_stride_head, const void* dout,
                            int64_t do_stride_tok, int64_t do_stride_head, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t n_seqs, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t Hq, int32_t Hkv, int32_t E, int32_t Ev,
                            int64_t total_q, int64_t total_k, int is_causal, const double* scale,
                            int enable_gqa, void* dq, int64_t dq_stride_tok, int64_t dq_stride_head,
                            void* dk, int64_t dk_stride_tok, int64_t dk_stride_head, void* dv,
                            int64_t dv_stride_tok, int64_t dv_stride_head, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (dtype != SDPA_F16 && dtype != SDPA_BF16 && dtype != SDPA_F32)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "dtype must be SDPA_F32, SDPA_F16 or SDPA_BF16");
    if (n_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || Hq < 0 || Hkv < 0 || E < 0 || Ev < 0 ||
        total_q < 0 || total_k < 0)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "sizes must be non-negative");
    if (Hq != Hkv) {
        if (!enable_gqa)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query has %d heads and key/value %d: pass enable_gqa",
                        Hq, Hkv);
        if (Hkv == 0 || Hq % Hkv != 0)
            return fail(SDPA_ERR_INVALID_ARGUMENT, "query heads (%d) must be a multiple of key/value heads (%d)",
                        Hq, Hkv);
    }
    if (n_seqs == 0 || Hq == 0 || (total_q == 0 && total_k == 0)) return ok();
    if (!cu_seqlens_q || !cu_seqlens_k)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "cu_seqlens_q and cu_seqlens_k must not be NULL");
    if (!forward_dims(E, Ev))
        return fail(SDPA_ERR_UNSUPPORTED, "head dims E=%d, Ev=%d: each must be a multiple of 8 up to 128", E, Ev);
    const void* ptrs[8] = {q, k, v, out, dout, dq, dk, dv};
    for (int i = 0; i < 8; ++i) {
        // zero-width rows (E = 0: q, k, dq, dk; Ev = 0: v, out, dout, dv) are never touched
        const bool width = (i == 0 || i == 1 || i == 5 || i == 6) ? E > 0 : Ev > 0;
        const bool need = width && ((i == 1 || i == 2 || i == 6 || i == 7) ? total_k > 0 : total_q > 0);
        if (need && !ptrs[i]) return fail(SDPA_ERR_INVALID_ARGUMENT, "data pointers must not be NULL");
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(SDPA_ERR_UNSUPPORTED, "packed tensors need 16-byte aligned base pointers");
    }
    if (total_q > 0 && !lse) return fail(SDPA_ERR_INVALID_ARGUMENT, "lse must not be NULL");
    const int64_t vec = 16 / elem_bytes(dtype);
    const int64_t strides[16] = {q_stride_tok, q_stride_head, k_stride_tok, k_stride_head, v_stride_tok,
                                 v_stride_head, o_stride_tok, o_stride_head, do_stride_tok, do_stride_head,
                                 dq_stride_tok, dq_stride_head, dk_stride_tok, dk_stride_head, dv_stride_tok,
                                 dv_stride_head};
    const bool swidth[8] = {E > 0, E > 0, Ev > 0, Ev > 0, Ev > 0, E > 0, E > 0, Ev > 0};
    for (int i = 0; i < 16; ++i)
        if (swidth[i / 2] && strides[i] % vec != 0)
            return fail(SDPA_ERR_UNSUPPORTED, "packed strides must be multiples of %lld elements", (long long)vec);
    double sc;
    sdpa_status st;
    if ((st = resolve_scale(scale, E, &sc)) != SDPA_OK) return st;
    const size_t need = (size_t)Hq * (size_t)total_q * sizeof(float) + 256;
    if (workspace_bytes < need || !workspace)
        return fail(SDPA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes needed, %zu given", need,
                    workspace_bytes);
    sdpa::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.dout = dout; p.lse = lse;
    p.dsum = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.q_sr = q_stride_tok; p.q_sh = q_stride_head;
    p.k_sr = k_stride_tok; p.k_sh = k_stride_head;
    p.v_sr = v_stride_tok; p.v_sh = v_stride_head;
    p.o_sr = o_stride_tok; p.o_sh = o_stride_head;
    p.do_sr = do_stride_tok; p.do_sh = do_stride_head;
    p.dq_sr = dq_stride_tok; p.dq_sh = dq_stride_head;
    p.dk_sr = dk_stride_tok; p.dk_sh = dk_stride_head;
    p.dv_sr = dv_stride_tok; p.dv_sh = dv_stride_head;
    p.lse_sh = lse_stride_head;
    p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
    p.total_q = total_q; p.total_k = total_k;
    p.B = n_seqs; p.Hq = Hq; p.Hkv = Hkv; p.group = Hq / Hkv;
    p.L = max_seqlen_q; p.S = max_seqlen_k;
    p.n_qtiles = (max_seqlen_q + 127) / 128;
    p.n_ktiles = (max_seqlen_k + 127) / 128;
    p.elem = dtype == SDPA_BF16 ? sdpa::ELEM_BF16 : dtype == SDPA_F16 ? sdpa::ELEM_F16 : sdpa::ELEM_F32;
    p.scale = (float)sc;
    p.e = E; p.ev = Ev;
    hipError_t e = matrix_core_backward(dtype, E, Ev)
                       ? sdpa::launch_backward(p, E, is_causal != 0, sdpa::MASK_NONE, true, (hipStream_t)stream)
                       : sdpa::launch_backward_vec(p, is_causal != 0, sdpa::MASK_NONE, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SDPA_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

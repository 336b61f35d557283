// Shared declarations of the attention kernels and their host launchers.
//
// Internal to libsdpa: the public interface is include/sdpa.h.  The forward
// kernels compute exact attention as the exactref.ai
// "scaled_dot_product_attention" page specifies it (section "Full
// specification"): softmax(scale * Q K^T + mask) V plus the per-row logsumexp;
// the backward kernels its gradients (section "backward").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

enum MaskKind { MASK_NONE = 0, MASK_FLOAT = 1, MASK_BOOL = 2 };
enum ElemType { ELEM_F32 = 0, ELEM_F16 = 1, ELEM_BF16 = 2 };

// One launch of the single-pass kernels (MFMA bf16/fp16 and VALU fp32).
// Strides are in elements.  Batched calls index (b, h, row); packed
// variable-length calls index (segment, h, token) with the token offset of a
// segment read from cu_q / cu_k.
struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const void* mask;     // float32 or uint8, (b, h, row, key); key stride 1
    const int* cu_q;      // varlen only: n_seqs + 1 offsets
    const int* cu_k;
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int64_t o_sb, o_sh, o_sr;
    int64_t lse_sb, lse_sh;  // lse element (b, h, i) at b*lse_sb + h*lse_sh + i (varlen: token index)
    int64_t m_sb, m_sh, m_sr;
    int64_t total_q, total_k;  // varlen: token counts, used to clamp offsets
    int B;                  // batch size (varlen: number of segments)
    int Hq, Hkv, group;     // group = Hq / Hkv
    int L, S;               // batched: lengths; varlen: max segment lengths
    int n_qtiles;
    int mask_vec;           // bit 0: vector mask loads allowed; bit 1: bool rows in whole 16-byte chunks
    int neg;                // the scale is negative: q is negated on load
    int dv;                 // value head dim Ev (== E except on the four-wave batched path)
    float scale_abs;        // |scale|
    float scale_log2;       // |scale| * log2(e)
    float scale;            // signed scale (fp32 kernel)
    // Paged key/value cache (block_table non-null; unmasked batched queries):
    // k_sb / v_sb = page stride, k_sh / v_sh = head stride, k_sr / v_sr = row
    // stride; key j of sequence b is row j mod 2^page_shift of page
    // block_table[b * bt_stride + (j >> page_shift)].  Sequence b holds
    // min(seq_lens[b], S, max_blocks << page_shift) keys, and its L query rows
    // are its last L positions (causal aligns bottom-right).
    const int* block_table;
    const int* seq_lens;
    int64_t bt_stride;
    int page_shift;
    int n_pages;
    int max_blocks;
    int e;                  // query/key head dim E (the padded instances read E of D columns)
};

// One launch of the split-KV decode kernel and of its merge pass.
struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    float* part_o;      // (B, Hq, L, n_splits, D) float32
    float* part_lse;    // (B, Hq, L, n_splits)    float32
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int64_t o_sb, o_sh, o_sr;
    int64_t lse_sb, lse_sh;
    int B, Hq, Hkv, group, L, S;
    int rows;           // L * group query rows share one key/value head
    int n_splits;
    int keys_per_split; // multiple of 128
    int neg;
    float scale_log2;   // |scale| * log2(e)
    // Paged cache (block_table non-null): k and v point at page pools with
    // k_sb / v_sb = page stride, k_sh / v_sh = head stride, k_sr / v_sr = row
    // stride; key j of sequence b is row j mod 2^page_shift of page
    // block_table[b * bt_stride + (j >> page_shift)]; sequence b holds
    // seq_lens[b] keys (clamped to S and to the table).  causal: the L new rows
    // are the sequence's last L positions (bottom-right alignment).
    const int* block_table;
    const int* seq_lens;
    int64_t bt_stride;
    int page_shift;
    int n_pages;
    int max_blocks;
    int causal;
    int dv;             // value head dim Ev (dense cache: may differ from E)
};

// One call of the backward kernels (bf16 / fp16).  dsum is the float32
// workspace of the per-row D = dO . O, laid out (b, h, i) contiguously.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    float* dsum;
    void* dq;
    void* dk;
    void* dv;
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int64_t o_sb, o_sh, o_sr;
    int64_t do_sb, do_sh, do_sr;
    int64_t dq_sb, dq_sh, dq_sr;
    int64_t dk_sb, dk_sh, dk_sr;
    int64_t dv_sb, dv_sh, dv_sr;
    int64_t lse_sb, lse_sh;
    int B, Hq, Hkv, group, L, S;
    int n_qtiles;   // 128-row query tiles
    int n_ktiles;   // 128-key tiles
    int elem;       // ELEM_BF16 or ELEM_F16 (the vector-ALU backward also ELEM_F32)
    float scale;    // signed
    // Optional mask, as in the forward: float32 bias or uint8 keep flags,
    // element (b, h, i, j) at b*m_sb + h*m_sh + i*m_sr + j (0 strides broadcast)
    const void* mask;
    int64_t m_sb, m_sh, m_sr;
    int mask_vec;   // rows allow vector loads (16-byte float / 8-byte bool runs)
    // Packed variable-length batches (cu_q non-null): B segments, row r of
    // segment b is token cu_q[b] + r (keys: cu_k[b] + j) with the _sr strides
    // per token; L, S bound the segment lengths; lse (h, token) at
    // h * lse_sh + token; the D workspace laid out (h, token).
    const int* cu_q;
    const int* cu_k;
    int64_t total_q, total_k;
    int e, ev;      // head dims of query/key rows and value rows
    // Optional dS^T store (batched calls, matrix-core kernels), 16-bit, in
    // panels of 128 queries: element (b, h, key j, query i) at
    // ((b * Hq + h) * ds_lp + (i & ~127)) * S + j * 128 + (i & 127), ds_lp a
    // multiple of 128 covering L, so 64 keys of one panel are 16 contiguous
    // KB.  Non-null: the dK/dV kernel writes dS there (zeros where no key is
    // kept) and dQ = scale dS K is formed from it.
    uint16_t* ds;
    int64_t ds_lp;
};

hipError_t launch_prefill_bf16(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                               hipStream_t stream);
hipError_t launch_prefill_f16(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                              hipStream_t stream);
hipError_t launch_prefill_f32(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                              hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int elem, int D, hipStream_t stream);
hipError_t launch_backward(const BwdParams& p, int D, bool causal, int mask, bool varlen, hipStream_t stream);
// The vector-ALU backward (any element type, head dims up to 128, Ev != E).
hipError_t launch_backward_vec(const BwdParams& p, bool causal, int mask, hipStream_t stream);

// Tile sizes the host needs for grids and workspace.
constexpr int kPrefillBlockM = 128;  // query rows per MFMA workgroup
constexpr int kF32BlockM = 64;       // query rows per fp32 workgroup
constexpr int kDecodeMaxRows = 16;   // query rows (L * group) per decode workgroup
constexpr int kDecodeKeyQuantum = 128;

}  // namespace sdpa

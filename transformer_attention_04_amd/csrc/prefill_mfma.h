// Single-pass attention forward for bf16 / fp16 inputs on gfx950 matrix cores:
// the four-wave kernel, and the dispatch of all bf16 / fp16 forward calls.
// Unmasked batched calls, float masks with aligned rows, bool masks whose
// rows are whole 16-byte chunks and queries against a paged cache with
// contiguous rows (packed rows too when the sequences bring about equal
// counts) go to the eight-wave kernel of prefill_pp.h; this kernel takes the
// other masks, packed variable-length batches, value rows of another width
// (Ev != E), head dims padded to a multiple of 32 (columns past E never read
// or written), and the other queries against a paged key/value cache
// (uneven packed rows, padded pool rows, more than 256 pages per sequence, a
// zero scale: pages read through the block table in 16-key groups, causal
// aligned bottom-right).
//
// Method: the blocked form of exact attention described on the khchao.com NN
// Lab page ("FlashAttention Tiling & Online Softmax Algorithm"): queries in
// blocks, keys and values streamed in blocks through on-chip memory, and a
// running (online) softmax so the score matrix never reaches HBM.  The result
// is the exact softmax(scale * Q K^T + mask) V of the exactref.ai
// "scaled_dot_product_attention" Full specification, up to rounding.
//
// gfx950 design
//  * A workgroup is 4 wavefronts of 64 lanes and owns 128 query rows; each
//    wavefront owns 32 rows.  Two workgroups share a compute unit (at most 256
//    registers per lane), so one workgroup's loads and softmax overlap the
//    other's matrix products.  Keys advance 64 per step through a
//    double-buffered LDS stage: K as rows, V transposed (V^T) so that both
//    matrix products read 16-byte runs along their contraction axis.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16
//    (A = 32 keys x 16 dims from LDS, B = 16 dims x 32 queries held in
//    registers for the whole loop).  Each lane then owns ONE query column and
//    16 keys of every 32-key block, so the row max and row sum of the online
//    softmax are in-lane reductions plus one exchange with lane ^ 32.
//  * K rows are placed in LDS in an order that swaps bits 2 and 3 of the key
//    index.  With that order the accumulator register r of lane l holds key
//    16*(r/8) + 8*(l/32) + r%8 of its block, which is exactly the k-slot order
//    the second product needs: O^T += V^T P^T takes P^T straight from the
//    score registers (rounded to bf16/fp16, as fused kernels do) with no LDS
//    round trip.  O^T also has one query per lane, so the rescale by
//    exp(m_old - m_new) is an in-lane multiply.
//  * The running max is raised only when a block's max exceeds it by more than
//    2^8 in the exponent; otherwise the old shift stays (weights stay <= 256)
//    and the O rescale is skipped.  Output and lse use the same shift as the
//    row sum, so the result is the same softmax.
//  * LDS layouts were chosen by measuring bank conflicts on gfx950 (the
//    SQ_LDS_BANK_CONFLICT counter over every access pattern of this kernel):
//    K rows padded to D+8 elements, and V^T rows of 64+8 elements with no
//    swizzle, read conflict-free; the transposing 8-byte V^T writes are
//    conflict-free when the 16 consecutive threads of a group take the 16
//    four-key groups of one 8-column chunk (rows 8 apart, columns 8 bytes
//    apart).
//  * Global memory is read and written through buffer resources sized to the
//    valid rows: rows past the end read as 0 and their stores are dropped, so
//    edge tiles need no branches.
//  * Causal: key blocks wholly above the diagonal are never loaded; wavefronts
//    whose rows all precede a block skip its products; masking by index runs
//    only on edge blocks.  Workgroups are dispatched heaviest query block first.
//  * Special rows: a row with no kept key keeps an unset shift, and ends with
//    output 0 and lse -inf; a NaN score makes exp NaN and the row NaN.
#pragma once

#include "attn_common.h"
#include "device_utils.h"
#include "prefill_pp.h"

#include <type_traits>

namespace sdpa {

// Wavefronts per SIMD: 3 where the registers allow it without spills (causal,
// unmasked, head dims <= 64: more wavefronts to overlap the softmax's vector
// work with the matrix products), else 2.
template <int D, int DV, bool CAUSAL, int MASK>
constexpr int kPrefillWaves = (D <= 64 && DV <= 64 && CAUSAL && MASK == MASK_NONE) ? 3 : 2;

// Packed batches (at most 4 x 64 segments): the g-th (segment, query tile)
// of one head in the order the workgroups take them.  Tile index qt is the
// level: every segment's tile qt_max first (segments in index order), then
// every segment's tile qt_max - 1, and so on, so that the tiles with the most
// key blocks start first, and the grid's workgroups past the last tile (the
// grid holds max tiles x segments) come last, where they end at once instead
// of holding places among the real tiles.  Each lane takes one segment of a
// chunk of 64 (one load of its two offsets); the walk down the levels is
// ballots and scalar counts.  Returns false when g is past the last tile;
// else the segment, its tile and its first token and row count.
constexpr int kPackedListMaxSegs = 256;
__device__ __forceinline__ bool packed_tile(const AttnParams& p, int g, int& seg, int& qt, int64_t& tok0,
                                            int& rows) {
    const int lane = threadIdx.x & 63;
    const int nch = (p.B + 63) / 64;
    int nt[kPackedListMaxSegs / 64];   // tiles of this lane's segment in each chunk
    int st[kPackedListMaxSegs / 64];   // its first token
    int ln[kPackedListMaxSegs / 64];   // its rows
#pragma unroll
    for (int c = 0; c < kPackedListMaxSegs / 64; ++c) {
        nt[c] = 0;
        st[c] = 0;
        ln[c] = 0;
        const int i = c * 64 + lane;
        if (c < nch && i < p.B) {
            const int64_t a = min(max((int64_t)p.cu_q[i], (int64_t)0), p.total_q);
            const int64_t e = min(max((int64_t)p.cu_q[i + 1], a), p.total_q);
            st[c] = (int)a;
            ln[c] = (int)min(e - a, (int64_t)p.L);
            nt[c] = (ln[c] + kPrefillBlockM - 1) / kPrefillBlockM;
        }
    }
    for (int t = p.n_qtiles - 1; t >= 0; --t) {
#pragma unroll
        for (int c = 0; c < kPackedListMaxSegs / 64; ++c) {
            if (c >= nch) break;
            const bool has = nt[c] > t;
            const unsigned long long m = __ballot(has);
            const int cnt = __popcll(m);
            if (g < cnt) {
                // the lane whose segment is the g-th set bit of m
                const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
                const int src = __builtin_ctzll(__ballot(has && rank == g));
                seg = c * 64 + src;
                qt = t;
                tok0 = __builtin_amdgcn_readlane(st[c], src);
                rows = __builtin_amdgcn_readlane(ln[c], src);
                return true;
            }
            g -= cnt;
        }
    }
    return false;
}

template <typename Tr, int D, int DV, bool CAUSAL, int MASK, bool VARLEN, bool PAGED = false,
          bool PADE = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kPrefillWaves<D, DV, CAUSAL, MASK>, kPrefillWaves<D, DV, CAUSAL, MASK>)))
void prefill_mfma_kernel(AttnParams p) {
    constexpr int BM = kPrefillBlockM;
    constexpr int BN = 64;
    constexpr int KS = D + 8;      // LDS row stride of the K tile, in 16-bit words
    constexpr int VS = BN + 8;     // LDS row stride of the V^T tile
    constexpr int KTILE = BN * KS;
    constexpr int VTILE = DV * VS;
    constexpr int STAGE = KTILE + VTILE;
    constexpr int NKK = D / 16;    // k-steps of the score product
    constexpr int NDB = DV / 32;   // 32-row blocks of O^T
    constexpr int KCH = BN * D / 8;          // 16-byte chunks of a K tile
    constexpr int KCH_T = KCH / 256;         // per thread
    constexpr int VIT = (DV / 8) * (BN / 4);  // V items: 8 columns x 4 keys
    static_assert(D % 32 == 0 && DV % 32 == 0 && KCH % 256 == 0, "head dims must be multiples of 32");
    static_assert(VIT <= 256, "one V item per thread");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lq = lane & 31;
    const int hh = lane >> 5;

    int qt, h, b;
    int64_t listed_a = 0;   // packed work list: the segment's first token and rows
    int listed_rows = 0;
    const bool listed = VARLEN && !PAGED && p.B <= kPackedListMaxSegs;
    if (listed) {
        // packed segments: a work list of the real tiles, the heaviest first
        h = (int)(blockIdx.x % p.Hq);
        if (!packed_tile(p, (int)(blockIdx.x / p.Hq), b, qt, listed_a, listed_rows)) return;
    } else {
        // Query tiles heaviest first; within one tile index, workgroups are
        // dealt to the 8 XCDs round-robin, so (when B * Hq is a multiple of 8)
        // XCD x takes the contiguous heads x * nbh / 8 .. : the query heads of
        // a key/value group share their keys in one L2, and each head stays
        // on one XCD for all its tiles.
        const int nbh = p.Hq * p.B;
        qt = p.n_qtiles - 1 - (int)(blockIdx.x / nbh);
        int bh = (int)(blockIdx.x % nbh);
        if ((nbh & 7) == 0) bh = (bh & 7) * (nbh >> 3) + (bh >> 3);
        h = bh % p.Hq;
        b = bh / p.Hq;
    }
    const int kvh = h / p.group;

    int Lb, Sb;
    int64_t qo, ko, vo, oo, lo, mo = 0;
    if (VARLEN && PAGED) {
        // packed new rows of sequence b (tokens cu_q[b] ..) against its paged keys
        const int64_t a = min(max((int64_t)p.cu_q[b], (int64_t)0), p.total_q);
        const int64_t e = min(max((int64_t)p.cu_q[b + 1], a), p.total_q);
        Lb = (int)min(e - a, (int64_t)p.L);
        Sb = min(max(p.seq_lens[b], 0), min(p.S, p.max_blocks << p.page_shift));
        qo = a * p.q_sr + (int64_t)h * p.q_sh;
        ko = (int64_t)kvh * p.k_sh;
        vo = (int64_t)kvh * p.v_sh;
        oo = a * p.o_sr + (int64_t)h * p.o_sh;
        lo = (int64_t)h * p.lse_sh + a;
    } else if (VARLEN) {
        const int64_t a = listed ? listed_a : min(max((int64_t)p.cu_q[b], (int64_t)0), p.total_q);
        const int64_t e = listed ? a + listed_rows : min(max((int64_t)p.cu_q[b + 1], a), p.total_q);
        const int64_t c = min(max((int64_t)p.cu_k[b], (int64_t)0), p.total_k);
        const int64_t d = min(max((int64_t)p.cu_k[b + 1], c), p.total_k);
        Lb = (int)min(e - a, (int64_t)p.L);
        Sb = (int)min(d - c, (int64_t)p.S);  // at most max_seqlen_k, as the backward
        qo = a * p.q_sr + (int64_t)h * p.q_sh;
        ko = c * p.k_sr + (int64_t)kvh * p.k_sh;
        vo = c * p.v_sr + (int64_t)kvh * p.v_sh;
        oo = a * p.o_sr + (int64_t)h * p.o_sh;
        lo = (int64_t)h * p.lse_sh + a;
    } else if (PAGED) {
        // keys of sequence b come page by page from the pool (offsets per tile)
        Lb = p.L;
        Sb = min(max(p.seq_lens[b], 0), min(p.S, p.max_blocks << p.page_shift));
        qo = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
        ko = (int64_t)kvh * p.k_sh;
        vo = (int64_t)kvh * p.v_sh;
        oo = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
        lo = (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;
    } else {
        Lb = p.L;
        Sb = p.S;
        qo = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
        ko = (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
        vo = (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;
        oo = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
        lo = (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh;
        mo = (int64_t)b * p.m_sb + (int64_t)h * p.m_sh;
    }
    const int q0 = qt * BM;
    if (q0 >= Lb) return;
    // causal: row i keeps key j <= i + coff (top-left, except bottom-right on a
    // paged cache, where the rows are the sequence's last Lb positions)
    const int coff = PAGED ? Sb - Lb : 0;
    const int kend = CAUSAL ? min(Sb, min(q0 + BM, Lb) + coff) : Sb;
    const int ntiles = ((PAGED ? max(kend, 0) : kend) + BN - 1) / BN;
    const int qrows = min(BM, Lb - q0);   // valid rows of this block
    const int wrow0 = wave * 32;          // first local row of this wavefront
    const int lrow = wrow0 + lq;          // local row this lane owns
    const int my_row = q0 + lrow;         // its query index
    const bool wave_has_rows = wrow0 < qrows;

    // Q^T operand, resident for the whole loop (negated when the scale is negative).
    // Row widths in bytes that bound the buffer resources.  The padded instances
    // must use E: with the padded width a row's range would reach into the next
    // rows (rows are only 2E bytes apart), and stores of rows past the tile's
    // valid rows would land in them instead of being dropped.
    const int qk_bytes = PADE ? p.e * 2 : D * 2;
    const int v_bytes = PADE ? p.dv * 2 : DV * 2;
    const int q_rs = (int)(p.q_sr * 2);
    const auto qrs = make_rsrc((const uint16_t*)p.q + qo + (int64_t)q0 * p.q_sr, (qrows - 1) * q_rs + qk_bytes);
    uint4 qreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        // padded head dim: columns from E on are not read (they load as 0)
        const int col = kk * 16 + hh * 8;
        qreg[kk] = buf_load16(qrs, (!PADE || col < p.e) ? lrow * q_rs + col * 2 : 0x7ffffff0);
    }
    wait_vmem_all();
    // negated after all loads have landed (a select per load would wait for each in turn)
    if (p.neg) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qreg[kk] = negate8(qreg[kk]);
    }

    const uint16_t* kbase = (const uint16_t*)p.k + ko;
    const uint16_t* vbase = (const uint16_t*)p.v + vo;
    const int k_rs = (int)(p.k_sr * 2);
    const int v_rs = (int)(p.v_sr * 2);
    uint4 kbuf[PAGED ? 4 : KCH_T];
    uint4 vbuf[4];
    // paged: bit g set when keys 16g .. 16g+15 of the last loaded tile lie on a
    // page outside the pool: they are not read, their K rows are stored as NaN
    // (so every row that keeps one of them is NaN) and their V rows as 0
    int bad_ld = 0;

    auto load_tile = [&](int key0) {
        if constexpr (PAGED) {
            // A tile is four 16-key groups, each inside one page (pages hold >= 16
            // keys), read through one buffer resource per group sized to its valid
            // rows: K load i takes group i (row 16i + tid/16, chunk tid%16), and
            // wavefront w takes group w of V (four-key run lane%4, chunk lane/4).
            int bad = 0;
            __amdgpu_buffer_rsrc_t kr[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int k16 = key0 + 16 * g;
                const int pg = k16 < Sb ? p.block_table[(int64_t)b * p.bt_stride + (k16 >> p.page_shift)] : 0;
                const bool okp = (unsigned)pg < (unsigned)p.n_pages;
                if (!okp && k16 < Sb) bad |= 1 << g;
                const int nv = okp ? min(16, Sb - k16) : 0;
                const int64_t row = (int64_t)(okp ? pg : 0) * p.k_sb + (int64_t)(k16 & ((1 << p.page_shift) - 1)) * p.k_sr;
                kr[g] = make_rsrc(kbase + row, nv > 0 ? (nv - 1) * k_rs + qk_bytes : 0);
            }
            bad_ld = bad;
            const int ch = tid & 15;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kbuf[i] = buf_load16(kr[i], (ch < D / 8 && (!PADE || ch * 8 < p.e)) ? (tid >> 4) * k_rs + ch * 16
                                                                                     : 0x7ffffff0);
            const int wv = __builtin_amdgcn_readfirstlane(wave);
            const int k16 = key0 + 16 * wv;
            const int pg = k16 < Sb ? p.block_table[(int64_t)b * p.bt_stride + (k16 >> p.page_shift)] : 0;
            const bool okp = (unsigned)pg < (unsigned)p.n_pages;
            const int nv = okp ? min(16, Sb - k16) : 0;
            const int64_t vrow = (int64_t)(okp ? pg : 0) * p.v_sb + (int64_t)(k16 & ((1 << p.page_shift) - 1)) * p.v_sr;
            const auto vr = make_rsrc(vbase + vrow, nv > 0 ? (nv - 1) * v_rs + v_bytes : 0);
            const int kq = lane & 3, dc = lane >> 2;
            const bool vin = dc < DV / 8 && (!PADE || dc * 8 < p.dv);
#pragma unroll
            for (int r = 0; r < 4; ++r) vbuf[r] = buf_load16(vr, vin ? (kq * 4 + r) * v_rs + dc * 16 : 0x7ffffff0);
            return;
        }
        const int rows = min(BN, Sb - key0);
        const auto kr = make_rsrc(kbase + (int64_t)key0 * p.k_sr, (rows - 1) * k_rs + qk_bytes);
        const auto vr = make_rsrc(vbase + (int64_t)key0 * p.v_sr, (rows - 1) * v_rs + v_bytes);
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (D / 8), col = (c % (D / 8)) * 8;
            kbuf[i] = buf_load16(kr, (!PADE || col < p.e) ? r * k_rs + col * 2 : 0x7ffffff0);
        }
        if (VIT == 256 || tid < VIT) {
            const int kg = tid % (BN / 4), dc = tid / (BN / 4);
            const bool vin = !PADE || dc * 8 < p.dv;
#pragma unroll
            for (int r = 0; r < 4; ++r) vbuf[r] = buf_load16(vr, vin ? (kg * 4 + r) * v_rs + dc * 16 : 0x7ffffff0);
        }
    };

    auto store_tile = [&](int stage) {
        uint16_t* Ks = smem + stage * STAGE;
        uint16_t* Vt = Ks + KTILE;
        if constexpr (PAGED) {
            // the load mapping of the paged branch of load_tile, same LDS layout
            if ((tid & 15) < D / 8) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * i + (tid >> 4);
                    const int row = (r & ~31) | swap_bits23(r & 31);
                    // all-ones halves are NaN in bf16 and fp16
                    const uint4 kv = ((bad_ld >> i) & 1) ? make_uint4(~0u, ~0u, ~0u, ~0u) : kbuf[i];
                    *(uint4*)(Ks + row * KS + (tid & 15) * 8) = kv;
                }
            }
            const int kg = 4 * wave + (lane & 3), dc = lane >> 2;
            if (dc < DV / 8) {
                const uint32_t* w0 = (const uint32_t*)&vbuf[0];
                const uint32_t* w1 = (const uint32_t*)&vbuf[1];
                const uint32_t* w2 = (const uint32_t*)&vbuf[2];
                const uint32_t* w3 = (const uint32_t*)&vbuf[3];
                uint16_t* base = Vt + kg * 4;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t lo = __builtin_amdgcn_perm(w1[j >> 1], w0[j >> 1], sel);
                    const uint32_t hi = __builtin_amdgcn_perm(w3[j >> 1], w2[j >> 1], sel);
                    *(uint2*)(base + (dc * 8 + j) * VS) = make_uint2(lo, hi);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (D / 8), col = (c % (D / 8)) * 8;
            const int row = (r & ~31) | swap_bits23(r & 31);
            *(uint4*)(Ks + row * KS + col) = kbuf[i];
        }
        if (VIT == 256 || tid < VIT) {
            const int kg = tid % (BN / 4), dc = tid / (BN / 4);
            const uint32_t* w0 = (const uint32_t*)&vbuf[0];
            const uint32_t* w1 = (const uint32_t*)&vbuf[1];
            const uint32_t* w2 = (const uint32_t*)&vbuf[2];
            const uint32_t* w3 = (const uint32_t*)&vbuf[3];
            uint16_t* base = Vt + kg * 4;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // keys kg*4 .. kg*4+3 of column dc*8 + j, as two packed pairs
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t lo = __builtin_amdgcn_perm(w1[j >> 1], w0[j >> 1], sel);
                const uint32_t hi = __builtin_amdgcn_perm(w3[j >> 1], w2[j >> 1], sel);
                *(uint2*)(base + (dc * 8 + j) * VS) = make_uint2(lo, hi);
            }
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    // Running shift in log2 units (-inf until the row sees a kept key) and this
    // lane's share of the row sum relative to it.
    float sh_run = kNegInf;
    float l_run = 0.f;    // row sum of the fp32 weights (for lse)
    float lr_run = 0.f;   // row sum of the weights rounded to 16 bits (normalises the output)
    // log2-domain logit = t * cfac, with t the raw score (or the fp32 logit when a
    // float mask is added).
    const float cfac = (MASK == MASK_FLOAT) ? kLog2e : p.scale_log2;

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int key0 = t * BN;
        if (t + 1 < ntiles) load_tile(key0 + BN);
        const uint16_t* Ks = smem + (t & 1) * STAGE;
        const uint16_t* Vt = Ks + KTILE;
        const bool active = wave_has_rows && (!CAUSAL || key0 <= q0 + wrow0 + 31 + coff);
        if (active) {
            f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint4 a = *(const uint4*)(Ks + (kb * 32 + lq) * KS + kk * 16 + hh * 8);
                    s[kb] = Tr::mfma32(as_vec8<Tr>(a), as_vec8<Tr>(qreg[kk]), s[kb]);
                }
            }
            // s[kb][8c + j] is the score of key key0 + 32kb + 16c + 8hh + j for query my_row.
            if (MASK == MASK_FLOAT) {
                // bias rows of this wavefront from key0 on; past the valid rows/keys reads 0
                const int mrow_bytes = (int)(p.m_sr * 4);
                const auto mr = make_rsrc((const float*)p.mask + mo + (int64_t)(q0 + wrow0) * p.m_sr + key0,
                                          ((qrows - 1 - wrow0) * (int)p.m_sr + (Sb - key0)) * 4);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int off = lq * mrow_bytes + (kb * 32 + c * 16 + hh * 8) * 4;
                        float bias[8];
                        if (p.mask_vec) {
                            const uint4 b0 = buf_load16(mr, off);
                            const uint4 b1 = buf_load16(mr, off + 16);
                            bias[0] = __uint_as_float(b0.x); bias[1] = __uint_as_float(b0.y);
                            bias[2] = __uint_as_float(b0.z); bias[3] = __uint_as_float(b0.w);
                            bias[4] = __uint_as_float(b1.x); bias[5] = __uint_as_float(b1.y);
                            bias[6] = __uint_as_float(b1.z); bias[7] = __uint_as_float(b1.w);
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j) bias[j] = __uint_as_float(buf_load4(mr, off + 4 * j));
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            s[kb][c * 8 + j] = fmaf(s[kb][c * 8 + j], p.scale_abs, bias[j]);
                    }
            }
            const bool edge = (key0 + BN > Sb) || (CAUSAL && key0 + BN - 1 > q0 + wrow0 + coff);
            // Register r of block kb holds local key kb*32 + (r/8)*16 + r%8 (+ 8hh + key0).
            // A key is kept when that local index is below `lim` (and the bool mask says so).
            uint32_t mbits = 0xffffffffu;
            if (MASK == MASK_BOOL) {
                const int mrow_bytes = (int)p.m_sr;
                const auto mr = make_rsrc((const uint8_t*)p.mask + mo + (int64_t)(q0 + wrow0) * p.m_sr + key0,
                                          (qrows - 1 - wrow0) * (int)p.m_sr + (Sb - key0));
                mbits = 0;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int off = lq * mrow_bytes + kb * 32 + c * 16 + hh * 8;
                        uint2 u;
                        if (p.mask_vec) {
                            u = buf_load8(mr, off);
                        } else {
                            u.x = u.y = 0;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                u.x |= buf_load1(mr, off + j) << (8 * j);
                                u.y |= buf_load1(mr, off + 4 + j) << (8 * j);
                            }
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const uint32_t byte = ((j < 4 ? u.x : u.y) >> (8 * (j & 3))) & 0xffu;
                            mbits |= (byte != 0 ? 1u : 0u) << (kb * 16 + c * 8 + j);
                        }
                    }
            }
            int lim = Sb - (key0 + hh * 8);
            if (CAUSAL) lim = min(lim, my_row + 1 + coff - (key0 + hh * 8));

            auto softmax_pv = [&](auto masked_tag) {
                constexpr bool MASKED = decltype(masked_tag)::value;
                if (MASKED) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int li = kb * 32 + (r >> 3) * 16 + (r & 7);
                            const bool ok = li < lim && ((mbits >> (kb * 16 + r)) & 1u);
                            s[kb][r] = ok ? s[kb][r] : kNegInf;
                        }
                }
                // row max over this lane's 32 scores: four short chains
                float m4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kb = i >> 1, r0 = (i & 1) * 8;
                    float m = fmaxf(s[kb][r0 + 0], s[kb][r0 + 1]);
#pragma unroll
                    for (int r = 2; r < 8; ++r) m = fmaxf(m, s[kb][r0 + r]);
                    m4[i] = m;
                }
                float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
                mx = pair32_max(mx);
                const float mxs = mx * cfac;                    // block max, log2 units
                const bool raise = mxs > sh_run + kLazyRescale;  // never for an all-masked block
                const float sh_new = raise ? mxs : sh_run;
                const float alpha = raise ? fast_exp2(sh_run - sh_new) : 1.f;
                sh_run = sh_new;
                const float shift = (sh_new == kNegInf) ? 0.f : sh_new;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float e = fast_exp2(fmaf(s[kb][r], cfac, -shift));
                        if (MASKED) e = (s[kb][r] == kNegInf) ? 0.f : e;
                        s[kb][r] = e;
                    }
                // this lane's share of the block's row sum, as a fixed tree
                float p8[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    p8[i] = (s[i >> 2][(i & 3) * 4 + 0] + s[i >> 2][(i & 3) * 4 + 1]) +
                            (s[i >> 2][(i & 3) * 4 + 2] + s[i >> 2][(i & 3) * 4 + 3]);
                const float tsum = ((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]));
                l_run = fmaf(l_run, alpha, tsum);
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
                }
                float r4[4];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        uint4 pb;
                        pb.x = Tr::pack2(s[kb][c * 8 + 0], s[kb][c * 8 + 1]);
                        pb.y = Tr::pack2(s[kb][c * 8 + 2], s[kb][c * 8 + 3]);
                        pb.z = Tr::pack2(s[kb][c * 8 + 4], s[kb][c * 8 + 5]);
                        pb.w = Tr::pack2(s[kb][c * 8 + 6], s[kb][c * 8 + 7]);
                        r4[kb * 2 + c] = Tr::sum2(pb.w, Tr::sum2(pb.z, Tr::sum2(pb.y, Tr::sum2(pb.x, 0.f))));
                        const int lchunk = kb * 4 + c * 2 + hh;
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int d = db * 32 + lq;
                            const uint4 a = *(const uint4*)(Vt + d * VS + lchunk * 8);
                            acc[db] = Tr::mfma32(as_vec8<Tr>(a), as_vec8<Tr>(pb), acc[db]);
                        }
                    }
                lr_run = fmaf(lr_run, alpha, (r4[0] + r4[1]) + (r4[2] + r4[3]));
            };
            if (edge || MASK == MASK_BOOL)
                softmax_pv(std::integral_constant<bool, true>{});
            else
                softmax_pv(std::integral_constant<bool, false>{});
        }
        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // Epilogue: O = O^T / l per lane (this lane's query), rounded to nearest-even.
    // The output divides by the sum of the same rounded weights that multiplied V
    // (a row dominated by one weight then keeps that weight's rounding out of
    // its output); lse takes the sum of the fp32 weights.
    const float l_tot = pair32_sum(l_run);
    const float lr_tot = pair32_sum(lr_run);
    const float inv = (lr_tot == 0.f) ? 0.f : 1.f / lr_tot;
    const int o_rs = (int)(p.o_sr * 2);
    const auto ors = make_rsrc((uint16_t*)p.o + oo + (int64_t)q0 * p.o_sr, (qrows - 1) * o_rs + v_bytes);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + g * 8 + hh * 4;
            uint2 st;
            st.x = Tr::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv);
            st.y = Tr::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
            if (!PADE || d < p.dv) buf_store8(st, ors, lrow * o_rs + d * 2);
        }
    if (hh == 0) {
        const float lse = (l_tot == 0.f) ? kNegInf : (sh_run + fast_log2(l_tot)) * kLn2;
        const auto lrs = make_rsrc(p.lse + lo + q0, qrows * 4);
        buf_store4(lse, lrs, lrow * 4);
    }
}

template <typename Tr, int D, int DV, bool CAUSAL, int MASK, bool VARLEN, bool PAGED = false,
          bool PADE = false>
hipError_t launch_prefill_one(const AttnParams& p, hipStream_t stream) {
    const long long grid = (long long)p.n_qtiles * p.Hq * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_mfma_kernel<Tr, D, DV, CAUSAL, MASK, VARLEN, PAGED, PADE>), dim3((unsigned)grid),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

// Value head dim DV != D: the four-wave kernel (its mask and packed-batch code
// reads scores only, so every mask kind and packed batches take any DV).
template <typename Tr, int D, int DV, bool CAUSAL>
hipError_t launch_prefill_dv_one(const AttnParams& p, int mask, bool varlen, hipStream_t s) {
    if (varlen)
        return mask == MASK_NONE ? launch_prefill_one<Tr, D, DV, CAUSAL, MASK_NONE, true>(p, s)
                                 : hipErrorInvalidValue;
    switch (mask) {
        case MASK_NONE: return launch_prefill_one<Tr, D, DV, CAUSAL, MASK_NONE, false>(p, s);
        case MASK_FLOAT: return launch_prefill_one<Tr, D, DV, CAUSAL, MASK_FLOAT, false>(p, s);
        case MASK_BOOL: return launch_prefill_one<Tr, D, DV, CAUSAL, MASK_BOOL, false>(p, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tr, int D>
hipError_t launch_prefill_dv(const AttnParams& p, bool causal, int mask, bool varlen, hipStream_t s) {
    if (p.block_table) return hipErrorInvalidValue;
    switch (p.dv) {
        case 64: if constexpr (D != 64) return causal ? launch_prefill_dv_one<Tr, D, 64, true>(p, mask, varlen, s)
                                                      : launch_prefill_dv_one<Tr, D, 64, false>(p, mask, varlen, s);
                 break;
        case 96: if constexpr (D != 96) return causal ? launch_prefill_dv_one<Tr, D, 96, true>(p, mask, varlen, s)
                                                      : launch_prefill_dv_one<Tr, D, 96, false>(p, mask, varlen, s);
                 break;
        case 128: if constexpr (D != 128) return causal ? launch_prefill_dv_one<Tr, D, 128, true>(p, mask, varlen, s)
                                                        : launch_prefill_dv_one<Tr, D, 128, false>(p, mask, varlen, s);
                  break;
    }
    return hipErrorInvalidValue;
}

template <typename Tr, int D>
hipError_t launch_prefill_d(const AttnParams& p, bool causal, int mask, bool varlen,
                            hipStream_t s) {
    if (p.dv != D) return launch_prefill_dv<Tr, D>(p, causal, mask, varlen, s);
    if (p.block_table) {
        // queries against a paged cache (more new rows than the split-KV decode
        // takes, or packed rows of several sequences)
        if (mask != MASK_NONE) return hipErrorInvalidValue;
        // the eight-wave kernel when the pool's rows are contiguous (its rows
        // of NaN for pages outside the pool have that stride), a sequence's
        // table row fits in four registers (256 pages) and the scale is not 0;
        // packed rows only when the sequences bring about equal counts (at
        // least 3/4 of n_seqs x max_seqlen_q rows): its workgroups take fixed
        // shares of the tiles, where the four-wave kernel's are handed out as
        // compute units free up
        const bool eight = p.scale_log2 > 0.f && p.k_sr == D && p.v_sr == D && p.max_blocks <= 256;
        if (varlen) {
            if (eight && 4 * p.total_q >= 3 * (int64_t)p.B * p.L)
                return causal ? launch_prefill_pp<Tr, D, true, MASK_NONE, true, true>(p, s)
                              : launch_prefill_pp<Tr, D, false, MASK_NONE, true, true>(p, s);
            return causal ? launch_prefill_one<Tr, D, D, true, MASK_NONE, true, true>(p, s)
                          : launch_prefill_one<Tr, D, D, false, MASK_NONE, true, true>(p, s);
        }
        if (eight)
            return causal ? launch_prefill_pp<Tr, D, true, MASK_NONE, true>(p, s)
                          : launch_prefill_pp<Tr, D, false, MASK_NONE, true>(p, s);
        return causal ? launch_prefill_one<Tr, D, D, true, MASK_NONE, false, true>(p, s)
                      : launch_prefill_one<Tr, D, D, false, MASK_NONE, false, true>(p, s);
    }
    if (varlen) {
        // packed segments keep the 128-row kernel: 256-row tiles waste more
        // rows on short segments
        if (mask != MASK_NONE) return hipErrorInvalidValue;
        return causal ? launch_prefill_one<Tr, D, D, true, MASK_NONE, true>(p, s)
                      : launch_prefill_one<Tr, D, D, false, MASK_NONE, true>(p, s);
    }
    switch (mask) {
        case MASK_NONE:
            // the eight-wave kernel masks scores with -inf and needs a positive
            // scale for exp2(-inf * scale) = 0; a zero scale stays here
            if (p.scale_log2 > 0.f)
                return causal ? launch_prefill_pp<Tr, D, true>(p, s)
                              : launch_prefill_pp<Tr, D, false>(p, s);
            return causal ? launch_prefill_one<Tr, D, D, true, MASK_NONE, false>(p, s)
                          : launch_prefill_one<Tr, D, D, false, MASK_NONE, false>(p, s);
        case MASK_FLOAT:
            // the eight-wave kernel moves the bias with 16-byte loads
            if (p.mask_vec)
                return causal ? launch_prefill_pp<Tr, D, true, MASK_FLOAT>(p, s)
                              : launch_prefill_pp<Tr, D, false, MASK_FLOAT>(p, s);
            return causal ? launch_prefill_one<Tr, D, D, true, MASK_FLOAT, false>(p, s)
                          : launch_prefill_one<Tr, D, D, false, MASK_FLOAT, false>(p, s);
        case MASK_BOOL:
            // the eight-wave kernel moves the mask in 16-byte chunks of whole
            // rows (bit 1 of mask_vec) and needs a positive scale (masked
            // scores are -inf before the scale is applied)
            if ((p.mask_vec & 2) && p.scale_log2 > 0.f)
                return causal ? launch_prefill_pp<Tr, D, true, MASK_BOOL>(p, s)
                              : launch_prefill_pp<Tr, D, false, MASK_BOOL>(p, s);
            return causal ? launch_prefill_one<Tr, D, D, true, MASK_BOOL, false>(p, s)
                          : launch_prefill_one<Tr, D, D, false, MASK_BOOL, false>(p, s);
    }
    return hipErrorInvalidValue;
}

// Other head dims (E and Ev multiples of 8 up to 128, E = 0 included, and Ev != E
// on a paged cache): the four-wave kernel at width W, the next multiple of 32
// of the larger one, reading E columns of Q and K and Ev of V (the rest load as
// 0, so the dot products only gain exact zeros) and writing Ev columns; every
// mask kind, packed batches and paged caches.
template <typename Tr, int W, bool CAUSAL>
hipError_t launch_prefill_pad_c(const AttnParams& p, int mask, bool varlen, hipStream_t s) {
    if (p.block_table) {
        if (mask != MASK_NONE) return hipErrorInvalidValue;
        return varlen ? launch_prefill_one<Tr, W, W, CAUSAL, MASK_NONE, true, true, true>(p, s)
                      : launch_prefill_one<Tr, W, W, CAUSAL, MASK_NONE, false, true, true>(p, s);
    }
    if (varlen)
        return mask == MASK_NONE ? launch_prefill_one<Tr, W, W, CAUSAL, MASK_NONE, true, false, true>(p, s)
                                 : hipErrorInvalidValue;
    switch (mask) {
        case MASK_NONE: return launch_prefill_one<Tr, W, W, CAUSAL, MASK_NONE, false, false, true>(p, s);
        case MASK_FLOAT: return launch_prefill_one<Tr, W, W, CAUSAL, MASK_FLOAT, false, false, true>(p, s);
        case MASK_BOOL: return launch_prefill_one<Tr, W, W, CAUSAL, MASK_BOOL, false, false, true>(p, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tr, int W>
hipError_t launch_prefill_pad(const AttnParams& p, bool causal, int mask, bool varlen, hipStream_t s) {
    return causal ? launch_prefill_pad_c<Tr, W, true>(p, mask, varlen, s)
                  : launch_prefill_pad_c<Tr, W, false>(p, mask, varlen, s);
}

template <typename Tr>
hipError_t launch_prefill_t(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                            hipStream_t s) {
    (void)D;
    const auto exact = [](int e) { return e == 64 || e == 96 || e == 128; };
    // exact instances; a paged cache with Ev != E takes the padded instance
    if (exact(p.e) && exact(p.dv) && !(p.block_table && p.e != p.dv)) {
        switch (p.e) {
            case 64: return launch_prefill_d<Tr, 64>(p, causal, mask, varlen, s);
            case 96: return launch_prefill_d<Tr, 96>(p, causal, mask, varlen, s);
            case 128: return launch_prefill_d<Tr, 128>(p, causal, mask, varlen, s);
        }
    }
    if (p.e < 0 || p.e > 128 || p.e % 8 != 0 || p.dv < 0 || p.dv > 128 || p.dv % 8 != 0)
        return hipErrorInvalidValue;
    switch ((max(max(p.e, p.dv), 1) + 31) / 32) {
        case 1: return launch_prefill_pad<Tr, 32>(p, causal, mask, varlen, s);
        case 2: return launch_prefill_pad<Tr, 64>(p, causal, mask, varlen, s);
        case 3: return launch_prefill_pad<Tr, 96>(p, causal, mask, varlen, s);
        case 4: return launch_prefill_pad<Tr, 128>(p, causal, mask, varlen, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sdpa

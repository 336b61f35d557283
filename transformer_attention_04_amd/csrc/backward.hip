// Gradients of exact attention for bf16 / fp16 inputs on gfx950 (CDNA4).
//
// What is computed: the exactref.ai "scaled_dot_product_attention.backward"
// section.  With P the attention weights, dP = dO V^T, D_i = sum_j P_ij dP_ij
// and dS = P * (dP - D):  dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q,
// dK and dV summed over the query heads that share a key/value head.  P is
// recomputed from the scores and the forward's logsumexp (P_ij = exp(l_ij -
// lse_i)), and D_i from the forward output (D_i = dO_i . O_i, equal to the
// definition's sum up to the rounding of O), as the blocked algorithm on the
// khchao.com NN Lab page keeps only O(N) state per row.
//
// Two schedules, chosen by the workspace the caller hands in:
//
// Stored dS (batched calls given the full workspace), three kernels:
//   bwd_dsum_kernel   D_i = dO_i . O_i in fp32 for every query row.
//   bwd_dkdv_kernel   one workgroup per 128 keys, over the query heads of the
//                     key/value head and their 64-row query blocks, with two
//                     roles per 32-key slice, sharing a SIMD: one wavefront
//                     computes S = Q K^T (one key per lane) and P, hands P to
//                     the other through LDS and accumulates dV^T += dO^T P;
//                     the other computes dP = dO V^T, then dS = P (dP - D) and
//                     dK^T += Q^T dS, and writes dS^T to the workspace in the
//                     16-bit input format.  P and dS are B operands from
//                     registers, dO^T and Q^T are read transposed from LDS.
//   bwd_dq_ds_kernel  one workgroup per 128 query rows: dQ^T += K^T dS^T from
//                     the stored dS^T, one matrix product per kept pair.
//   Four products in the dK/dV kernel and one in the dQ kernel: the 5 of the
//   definition (S, dP, dV, dK, dQ) per kept (query, key) pair and head
//   dimension, at the price of writing and reading dS^T once.
//
// Recomputed dS (packed batches, or a workspace holding only D), two kernels:
//   bwd_dq_kernel     one workgroup per 128 query rows (4 wavefronts x 32);
//                     first D_i = dO_i . O_i from the dO rows it holds and the
//                     O rows in the same layout (written to the workspace for
//                     the second kernel, which runs after it); for each 64-key
//                     block, S^T = K Q^T and dP^T = V dO^T on the matrix cores
//                     (the transposed score layout of the forward kernels, one
//                     query per lane), P^T and dS^T in registers, then
//                     dQ^T += K^T dS^T with dS^T as the B operand straight from
//                     the score registers and K^T read from LDS with the
//                     transposing ds_read_b64_tr_b16.
//   bwd_dkdv_kernel   as above, without the dS^T stores.
//   S and dP are then computed twice (once per kernel), 7 products per kept
//   pair and head dimension.
// Both schedules compute D, P and dS with the same arithmetic, so they give
// bit-identical gradients.  No atomics: each gradient element has one owner,
// and every wavefront fits in 256 registers (two per SIMD).
//
// Optional masks, as in the forward: a float32 bias enters the logit as
// scale * s + bias, a bool mask sets P = 0 on the keys it drops; the dQ kernel
// reads its row's mask in 8-key runs, the dK/dV kernel down its key's column.
// A row whose forward kept no key (lse -inf) is read with lse 0, so all its
// weights are exp(-inf) = 0 and it contributes nothing.  Packed
// variable-length batches (block-diagonal mask) take each segment's first
// token and lengths from cu_seqlens and address rows by token.
//
// LDS tiles are row-major with 8 elements of padding per row.  A product's
// row m (the row a lane reads for the first product, and so the row of the
// result) is stored at position rowpos(m): m's place within its group of 16
// rows, written 4a + b, becomes 4b + a.  Then the 16 lanes of a 16-byte row
// read touch 16 distinct positions of one group (distinct 4-bank groups at
// these strides), and the four rows of a transposing read (4 consecutive
// product rows) sit 4 positions apart, i.e. 16 banks apart, so the 32 lanes
// of one 8-byte transposing read hit 64 distinct banks.  Natural row r is
// product row swap23(r) (bits 2 and 3 of its index within a 32-row group
// swapped): then register r of lane l of a 32x32 product tile holds natural
// row 16(r/8) + 8(l/32) + r%8 of its group, which is exactly the k-slot order
// of a B operand.
#include "attn_common.h"
#include "device_utils.h"

#include <type_traits>

namespace sdpa {

namespace {

__device__ __forceinline__ int bwd_swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// LDS position of product row m (the 4 x 4 transpose of m's place in its 16-row group)
__device__ __forceinline__ int bwd_rowpos(int m) { return (m & ~15) | ((m & 3) << 2) | ((m >> 2) & 3); }
// LDS position of natural row r: product row swap23(r)
__device__ __forceinline__ int bwd_pos(int r) { return bwd_rowpos((r & ~31) | bwd_swap23(r & 31)); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// A operand X^T (32 columns of X as rows, 16 rows of X as k-slots) of one
// 16-row chunk c of a row-major tile X[pos][RS] (16-bit words): lane l gets
// column col0 + (l & 31) and natural rows 16c + 8(l/32) + 0..7, in two
// transposing reads of 4 rows each.
template <int RS>
__device__ __forceinline__ uint4 read_tr(const uint16_t* tile, int c, int col0, int lane) {
    const int i = lane & 15, g = (lane >> 4) & 1, hh = lane >> 5;
    const int col = col0 + 16 * g + 4 * (i & 3);
    const uint16_t* a0 = tile + bwd_rowpos(16 * c + 4 * hh + (i >> 2)) * RS + col;
    const uint16_t* a1 = tile + bwd_rowpos(16 * c + 8 + 4 * hh + (i >> 2)) * RS + col;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(uint32_t)(uintptr_t)a0);
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(uintptr_t)(uint32_t)(uintptr_t)a1);
    uint4 u;
    u.x = __builtin_bit_cast(uint2, lo).x;
    u.y = __builtin_bit_cast(uint2, lo).y;
    u.z = __builtin_bit_cast(uint2, hi).x;
    u.w = __builtin_bit_cast(uint2, hi).y;
    return u;
}

// ------------------------------------------------------------- D = dO . O

// D_i = dO_i . O_i in fp32 for every query row of a batched call (the
// schedule that stores dS needs it before the dK/dV kernel).  The same
// arithmetic as the dQ kernel's own D: each half of a 32-lane pair takes
// elements 16kk + 8hh .. +7 of its row in order, products accumulated by
// fmaf, the two halves added; so both schedules see the same D.  The 128 rows
// of O and dO travel to LDS first with whole rows per load instruction (a
// lane-per-row load would touch 32 rows per instruction).
template <typename Tr, int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdParams p) {
    constexpr int NKK = D / 16;
    constexpr int RW = D + 8;              // LDS row stride, 16-bit words
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int NCH_T = 128 * CPR / 256; // chunks per thread and tensor
    static_assert(128 * CPR % 256 == 0, "chunks per thread");
    __shared__ __attribute__((aligned(16))) uint16_t so[128 * RW];
    __shared__ __attribute__((aligned(16))) uint16_t sg[128 * RW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hh = lane >> 5;
    const int nbh = p.Hq * p.B;
    const int qt = (int)(blockIdx.x / nbh), bh = (int)(blockIdx.x % nbh);
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int q0 = qt * 128;
    if (q0 >= p.L) return;
    const int qrows = min(128, p.L - q0);
    const int lrow = wave * 32 + lq;
    const int o_rs = (int)(p.o_sr * 2), do_rs = (int)(p.do_sr * 2);
    const auto ors = make_rsrc((const uint16_t*)p.o + (int64_t)b * p.o_sb + h * p.o_sh + (int64_t)q0 * p.o_sr,
                               (qrows - 1) * o_rs + D * 2);
    const auto grs = make_rsrc((const uint16_t*)p.dout + (int64_t)b * p.do_sb + h * p.do_sh + (int64_t)q0 * p.do_sr,
                               (qrows - 1) * do_rs + D * 2);
    uint4 ov[NCH_T], gv[NCH_T];
#pragma unroll
    for (int i = 0; i < NCH_T; ++i) {
        const int c = tid + 256 * i, r = c / CPR, col = (c % CPR) * 8;
        ov[i] = buf_load16(ors, r * o_rs + col * 2);   // rows past the last read 0
        gv[i] = buf_load16(grs, r * do_rs + col * 2);
    }
#pragma unroll
    for (int i = 0; i < NCH_T; ++i) {
        const int c = tid + 256 * i, r = c / CPR, col = (c % CPR) * 8;
        *(uint4*)(so + r * RW + col) = ov[i];
        *(uint4*)(sg + r * RW + col) = gv[i];
    }
    __syncthreads();
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const uint4 o = *(const uint4*)(so + lrow * RW + kk * 16 + hh * 8);
        const uint4 g = *(const uint4*)(sg + lrow * RW + kk * 16 + hh * 8);
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dpart = fmaf(Tr::to_f32(ow[j] & 0xffffu), Tr::to_f32(gw[j] & 0xffffu), dpart);
            dpart = fmaf(Tr::to_f32(ow[j] >> 16), Tr::to_f32(gw[j] >> 16), dpart);
        }
    }
    const float dfull = pair32_sum(dpart);  // every lane takes part in the exchange
    if (lrow < qrows && hh == 0) p.dsum[((int64_t)b * p.Hq + h) * p.L + q0 + lrow] = dfull;
}


// ------------------------------------------------------------------- dQ

// Mask values of 8 consecutive keys starting at byte offset off of a
// range-checked mask resource: float32 bias (MASK_FLOAT) into b[0..7], or keep
// flags (MASK_BOOL, any nonzero byte keeps) into bits 0..7 of the result.
template <int MASK>
__device__ __forceinline__ uint32_t bwd_mask8(__amdgpu_buffer_rsrc_t r, int off, bool vec, float* b) {
    if constexpr (MASK == MASK_FLOAT) {
        if (vec) {
            const uint4 b0 = buf_load16(r, off), b1 = buf_load16(r, off + 16);
            b[0] = __uint_as_float(b0.x); b[1] = __uint_as_float(b0.y);
            b[2] = __uint_as_float(b0.z); b[3] = __uint_as_float(b0.w);
            b[4] = __uint_as_float(b1.x); b[5] = __uint_as_float(b1.y);
            b[6] = __uint_as_float(b1.z); b[7] = __uint_as_float(b1.w);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = __uint_as_float(buf_load4(r, off + 4 * j));
        }
        return 0xffu;
    } else {
        uint2 u;
        if (vec) {
            u = buf_load8(r, off);
        } else {
            u.x = u.y = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u.x |= buf_load1(r, off + j) << (8 * j);
                u.y |= buf_load1(r, off + 4 + j) << (8 * j);
            }
        }
        uint32_t bits = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) bits |= ((((j < 4 ? u.x : u.y) >> (8 * (j & 3))) & 0xffu) != 0 ? 1u : 0u) << j;
        return bits;
    }
}

// Segment b of a packed batch: first row a and key c, lengths Lb and Sb
// (offsets clamped to the packed totals, lengths to the launch's L and S).
__device__ __forceinline__ void bwd_segment(const BwdParams& p, int b, int64_t& a, int& Lb, int64_t& c, int& Sb) {
    const int64_t a0 = min(max((int64_t)p.cu_q[b], (int64_t)0), p.total_q);
    const int64_t e0 = min(max((int64_t)p.cu_q[b + 1], a0), p.total_q);
    const int64_t c0 = min(max((int64_t)p.cu_k[b], (int64_t)0), p.total_k);
    const int64_t d0 = min(max((int64_t)p.cu_k[b + 1], c0), p.total_k);
    a = a0;
    c = c0;
    Lb = (int)min(e0 - a0, (int64_t)p.L);
    Sb = (int)min(d0 - c0, (int64_t)p.S);
}

template <typename Tr, int D, bool CAUSAL, int MASK = MASK_NONE, bool VARLEN = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
    static_assert(!(VARLEN && MASK != MASK_NONE), "packed batches take no mask");
    constexpr int BM = 128, BN = 64;
    constexpr int RS = D + 8;            // LDS row stride, 16-bit words
    constexpr int TILE = BN * RS;        // one K or V block
    constexpr int STAGE = 2 * TILE;
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int NCH = BN * D / 8;      // 16-byte chunks per block
    constexpr int NCH_T = NCH / 256;     // per thread
    static_assert(NCH % 256 == 0, "chunks per thread");
    // operand reads issued in groups ahead of their products, where the registers allow
    constexpr bool kBatchReads = D < 128;                     // score and dP operands
    constexpr bool kBatchTr = MASK == MASK_NONE || D < 128;   // dQ product operands
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar
    const int lq = lane & 31, hh = lane >> 5;
    const int nbh = p.Hq * p.B;
    const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / nbh);  // heaviest (causal) first
    const int bh = (int)(blockIdx.x % nbh);
    const int h = bh % p.Hq, b = bh / p.Hq, kvh = h / p.group;
    int Lb = p.L, Sb = p.S;
    int64_t qa = 0, kc = 0;  // packed batches: first token of segment b's rows and keys
    if constexpr (VARLEN) bwd_segment(p, b, qa, Lb, kc, Sb);
    const int64_t q_b = VARLEN ? qa * p.q_sr : b * p.q_sb, do_b = VARLEN ? qa * p.do_sr : b * p.do_sb;
    const int64_t k_b = VARLEN ? kc * p.k_sr : b * p.k_sb, v_b = VARLEN ? kc * p.v_sr : b * p.v_sb;
    const int64_t dq_b = VARLEN ? qa * p.dq_sr : b * p.dq_sb;
    const int q0 = qt * BM;
    if (q0 >= Lb) return;
    const int qrows = min(BM, Lb - q0);
    const int wrow0 = wave * 32;
    const int my_row = q0 + wrow0 + lq;
    const bool wave_has_rows = wrow0 < qrows;
    const int kend = CAUSAL ? min(Sb, q0 + BM) : Sb;
    const int ntiles = (kend + BN - 1) / BN;

    // Q^T and dO^T operands (lane: query lq, elements 16kk + 8hh .. +7)
    const int q_rs = (int)(p.q_sr * 2), do_rs = (int)(p.do_sr * 2);
    const auto qrs = make_rsrc((const uint16_t*)p.q + q_b + h * p.q_sh + (int64_t)q0 * p.q_sr,
                               (qrows - 1) * q_rs + D * 2);
    const auto gdrs = make_rsrc((const uint16_t*)p.dout + do_b + h * p.do_sh + (int64_t)q0 * p.do_sr,
                                (qrows - 1) * do_rs + D * 2);
    const int lrow = wrow0 + lq;
    uint4 qreg[NKK], dreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        qreg[kk] = buf_load16(qrs, lrow * q_rs + (kk * 16 + hh * 8) * 2);
        dreg[kk] = buf_load16(gdrs, lrow * do_rs + (kk * 16 + hh * 8) * 2);
    }
    // D_i = dO_i . O_i for this lane's row: O in the layout of dO, fp32 products
    // over the lane's half of the row, then the other half from lane ^ 32
    const int o_rs = (int)(p.o_sr * 2);
    const int64_t o_b = VARLEN ? qa * p.o_sr : b * p.o_sb;
    const auto ors_in = make_rsrc((const uint16_t*)p.o + o_b + h * p.o_sh + (int64_t)q0 * p.o_sr,
                                  (qrows - 1) * o_rs + D * 2);
    float dpart = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        const uint4 o = buf_load16(ors_in, lrow * o_rs + (kk * 16 + hh * 8) * 2);
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
        const uint32_t gw[4] = {dreg[kk].x, dreg[kk].y, dreg[kk].z, dreg[kk].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dpart = fmaf(Tr::to_f32(ow[j] & 0xffffu), Tr::to_f32(gw[j] & 0xffffu), dpart);
            dpart = fmaf(Tr::to_f32(ow[j] >> 16), Tr::to_f32(gw[j] >> 16), dpart);
        }
    }
    const int64_t rowid = VARLEN ? (int64_t)h * p.total_q + qa : ((int64_t)b * p.Hq + h) * p.L;
    const int64_t lse_b = VARLEN ? h * p.lse_sh + qa : b * p.lse_sb + h * p.lse_sh;
    const bool row_ok = my_row < Lb;
    float lse2 = row_ok ? p.lse[lse_b + my_row] * kLog2e : 0.f;
    // a masked row with no kept key (lse -inf) has P = 0: exp2(-inf - 0)
    if (MASK != MASK_NONE && lse2 == kNegInf) lse2 = 0.f;
    const float dfull = pair32_sum(dpart);  // every lane takes part in the exchange
    const float drow = row_ok ? dfull : 0.f;
    // the dK/dV kernel, launched after this one, reads D from the workspace
    if (row_ok && hh == 0) p.dsum[rowid + my_row] = drow;
    const float c2 = p.scale * kLog2e;  // signed
    // All of the above has landed before the loop: otherwise the first uses in
    // the loop would wait (in every iteration) for the loads issued after them,
    // the next block's prefetch included.
    wait_vmem_all();

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

    const uint16_t* kbase = (const uint16_t*)p.k + k_b + kvh * p.k_sh;
    const uint16_t* vbase = (const uint16_t*)p.v + v_b + kvh * p.v_sh;
    const int k_rs = (int)(p.k_sr * 2), v_rs = (int)(p.v_sr * 2);
    uint4 kbuf[NCH_T], vbuf[NCH_T];
    auto load_tile = [&](int key0) {
        const int rows = min(BN, Sb - key0);
        const auto kr = make_rsrc(kbase + (int64_t)key0 * p.k_sr, (rows - 1) * k_rs + D * 2);
        const auto vr = make_rsrc(vbase + (int64_t)key0 * p.v_sr, (rows - 1) * v_rs + D * 2);
#pragma unroll
        for (int i = 0; i < NCH_T; ++i) {
            const int ch = tid + 256 * i, r = ch / (D / 8), col = (ch % (D / 8)) * 8;
            kbuf[i] = buf_load16(kr, r * k_rs + col * 2);
            vbuf[i] = buf_load16(vr, r * v_rs + col * 2);
        }
    };
    auto store_tile = [&](int stage) {
        uint16_t* Ks = smem + stage * STAGE;
        uint16_t* Vs = Ks + TILE;
#pragma unroll
        for (int i = 0; i < NCH_T; ++i) {
            const int ch = tid + 256 * i, r = ch / (D / 8), col = (ch % (D / 8)) * 8;
            *(uint4*)(Ks + bwd_pos(r) * RS + col) = kbuf[i];
            *(uint4*)(Vs + bwd_pos(r) * RS + col) = vbuf[i];
        }
    };

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int key0 = t * BN;
        if (t + 1 < ntiles) load_tile(key0 + BN);
        const uint16_t* Ks = smem + (t & 1) * STAGE;
        const uint16_t* Vs = Ks + TILE;
        const bool active = wave_has_rows && (!CAUSAL || key0 <= q0 + wrow0 + 31);
        if (active) {
            f32x16_t s[2] = {f32x16_t{}, f32x16_t{}}, dp[2] = {f32x16_t{}, f32x16_t{}};
            if constexpr (kBatchReads) {
                // the operand reads of two head-dim chunks (8 reads) issued together
#pragma unroll
                for (int k0 = 0; k0 < NKK; k0 += 2) {
                    uint4 ka[2][2], va[2][2];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            ka[i][kb] = *(const uint4*)(Ks + bwd_rowpos(kb * 32 + lq) * RS + (k0 + i) * 16 + hh * 8);
                            va[i][kb] = *(const uint4*)(Vs + bwd_rowpos(kb * 32 + lq) * RS + (k0 + i) * 16 + hh * 8);
                        }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            s[kb] = Tr::mfma32(as_vec8<Tr>(ka[i][kb]), as_vec8<Tr>(qreg[k0 + i]), s[kb]);
                            dp[kb] = Tr::mfma32(as_vec8<Tr>(va[i][kb]), as_vec8<Tr>(dreg[k0 + i]), dp[kb]);
                        }
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const uint4 ka = *(const uint4*)(Ks + bwd_rowpos(kb * 32 + lq) * RS + kk * 16 + hh * 8);
                        const uint4 va = *(const uint4*)(Vs + bwd_rowpos(kb * 32 + lq) * RS + kk * 16 + hh * 8);
                        s[kb] = Tr::mfma32(as_vec8<Tr>(ka), as_vec8<Tr>(qreg[kk]), s[kb]);
                        dp[kb] = Tr::mfma32(as_vec8<Tr>(va), as_vec8<Tr>(dreg[kk]), dp[kb]);
                    }
            }
            // register r of block kb: key key0 + 32kb + 16(r/8) + 8hh + r%8, query my_row
            const bool edge = (key0 + BN > Sb) || (CAUSAL && key0 + BN - 1 > q0 + wrow0);
            // keys of register r are kept below lim (every key of a block inside the limits)
            int lim = Sb - (key0 + hh * 8);
            if (CAUSAL) lim = min(lim, my_row + 1 - (key0 + hh * 8));
            if (!edge) lim = BN;
            uint4 pb[4];
            constexpr int MES = MASK == MASK_FLOAT ? 4 : 1;  // bytes per mask element
            // this wave's rows of the mask from key key0 on (unused without a mask)
            const auto mr = make_rsrc(
                MASK == MASK_NONE ? p.mask
                                  : (const char*)p.mask + ((int64_t)b * p.m_sb + (int64_t)h * p.m_sh +
                                                           (int64_t)(q0 + wrow0) * p.m_sr + key0) * MES,
                MASK == MASK_NONE ? 0 : ((qrows - 1 - wrow0) * (int)p.m_sr + (Sb - key0)) * MES);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float ds[16];
                float mb[16];       // float mask: bias of register r
                uint32_t mk = ~0u;  // bool mask: keep bit of register r
                if constexpr (MASK != MASK_NONE) {
                    mk = 0;
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        mk |= bwd_mask8<MASK>(mr, (lq * (int)p.m_sr + kb * 32 + c * 16 + hh * 8) * MES, p.mask_vec != 0,
                                              mb + 8 * c) << (8 * c);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pv;
                    if constexpr (MASK == MASK_FLOAT)
                        pv = fast_exp2(fmaf(fmaf(s[kb][r], p.scale, mb[r]), kLog2e, -lse2));
                    else
                        pv = fast_exp2(fmaf(s[kb][r], c2, -lse2));
                    if constexpr (MASK == MASK_BOOL) pv = ((mk >> r) & 1u) ? pv : 0.f;
                    pv = (kb * 32 + (r >> 3) * 16 + (r & 7) < lim) ? pv : 0.f;
                    ds[r] = pv * (dp[kb][r] - drow);
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    pb[kb * 2 + c].x = Tr::pack2(ds[c * 8 + 0], ds[c * 8 + 1]);
                    pb[kb * 2 + c].y = Tr::pack2(ds[c * 8 + 2], ds[c * 8 + 3]);
                    pb[kb * 2 + c].z = Tr::pack2(ds[c * 8 + 4], ds[c * 8 + 5]);
                    pb[kb * 2 + c].w = Tr::pack2(ds[c * 8 + 6], ds[c * 8 + 7]);
                }
            }
            // dQ^T (rows e, columns queries) += K^T dS^T over the block's 4 key chunks
            if constexpr (kBatchTr) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint4 a[NDB];   // one chunk's reads together
#pragma unroll
                    for (int db = 0; db < NDB; ++db) a[db] = read_tr<RS>(Ks, c, db * 32, lane);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[db] = Tr::mfma32(as_vec8<Tr>(a[db]), as_vec8<Tr>(pb[c]), acc[db]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const uint4 a = read_tr<RS>(Ks, c, db * 32, lane);
                        acc[db] = Tr::mfma32(as_vec8<Tr>(a), as_vec8<Tr>(pb[c]), acc[db]);
                    }
            }
        }
        // the other stage was last read a step ago, before the last barrier
        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // dQ = scale * dQ^T, rounded to nearest-even; lane: query lrow, e = 32db + 8g + 4hh + 0..3
    const int dq_rs = (int)(p.dq_sr * 2);
    const auto ors = make_rsrc((uint16_t*)p.dq + dq_b + h * p.dq_sh + (int64_t)q0 * p.dq_sr,
                               (qrows - 1) * dq_rs + D * 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + g * 8 + hh * 4;
            uint2 st;
            st.x = Tr::pack2(acc[db][4 * g + 0] * p.scale, acc[db][4 * g + 1] * p.scale);
            st.y = Tr::pack2(acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
            buf_store8(st, ors, lrow * dq_rs + d * 2);
        }
}

// ---------------------------------------------------------- dQ from dS^T

// dQ = scale dS K for batched calls whose dK/dV kernel stored dS^T (one
// workgroup per 128 query rows, 4 wavefronts x 32 rows): per 64-key block, K
// and the block's dS^T rows (keys) x 128 query columns (16 contiguous KB of
// the query tile's panel) travel to LDS through registers, and dQ^T += K^T
// dS^T with both operands read transposed by ds_read_b64_tr_b16: one matrix
// product per (query, key) pair where the recomputing dQ kernel needs three
// (S, dP and this one).  The kernel moves more bytes per product than it
// computes, so the loads run two blocks ahead (two register sets, used in
// turn), which keeps twice as many bytes in flight as a one-block prefetch.
// dS^T is stored for every key block up to the causal limit of a 128-row tile
// (zeros where no key is kept), so no mask, scale or softmax work is left.
template <typename Tr, int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_ds_kernel(BwdParams p) {
    constexpr int BM = 128, BN = 64;
    constexpr int RS = D + 8;            // K tile row stride, 16-bit words
    constexpr int RQ = BM + 8;           // dS^T tile row stride
    constexpr int KTILE = BN * RS, STILE = BN * RQ;
    constexpr int STAGE = KTILE + STILE;
    constexpr int NDB = D / 32;
    constexpr int KCH_T = BN * D / 8 / 256;   // 16-byte K chunks per thread
    constexpr int SCH_T = BN * BM / 8 / 256;  // 16-byte dS^T chunks per thread
    static_assert(BN * D / 8 % 256 == 0 && BN * BM / 8 % 256 == 0, "chunks per thread");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, hh = lane >> 5;
    const int nbh = p.Hq * p.B;
    const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / nbh);  // heaviest (causal) first
    const int bh = (int)(blockIdx.x % nbh);
    const int h = bh % p.Hq, b = bh / p.Hq, kvh = h / p.group;
    const int q0 = qt * BM;
    if (q0 >= p.L) return;
    const int qrows = min(BM, p.L - q0);
    const int kend = CAUSAL ? min(p.S, q0 + BM) : p.S;
    const int ntiles = (kend + BN - 1) / BN;

    const uint16_t* kbase = (const uint16_t*)p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const uint16_t* sbase = p.ds + (((int64_t)b * p.Hq + h) * p.ds_lp + q0) * p.S;  // panel of q0
    const int k_rs = (int)(p.k_sr * 2);
    struct Tile {
        uint4 k[KCH_T], s[SCH_T];
    };
    // block t into registers; a block past the last has empty ranges (its
    // loads read nothing), so every step issues the same loads
    auto load_tile = [&](int t, Tile& r) {
        const int key0 = t < ntiles ? t * BN : 0;
        const int rows = t < ntiles ? min(BN, p.S - key0) : 0;
        const auto kr = make_rsrc(kbase + (int64_t)key0 * p.k_sr, rows > 0 ? (rows - 1) * k_rs + D * 2 : 0);
        const auto sr = make_rsrc(sbase + (int64_t)key0 * BM, rows * BM * 2);
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i, rr = c / (D / 8), col = (c % (D / 8)) * 8;
            r.k[i] = buf_load16(kr, rr * k_rs + col * 2);
        }
#pragma unroll
        for (int i = 0; i < SCH_T; ++i) r.s[i] = buf_load16_nt(sr, (tid + 256 * i) * 16);
    };
    auto store_tile = [&](int stage, const Tile& r) {
        uint16_t* Ks = smem + stage * STAGE;
        uint16_t* Ds = Ks + KTILE;
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i, rr = c / (D / 8), col = (c % (D / 8)) * 8;
            *(uint4*)(Ks + bwd_pos(rr) * RS + col) = r.k[i];
        }
#pragma unroll
        for (int i = 0; i < SCH_T; ++i) {
            const int c = tid + 256 * i, rr = c / (BM / 8), col = (c % (BM / 8)) * 8;
            *(uint4*)(Ds + bwd_pos(rr) * RQ + col) = r.s[i];
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    // Transposed operand reads (as read_tr): lane (i = l & 15, g, hh) reads
    // 4 rows from tile row rowpos(16c + 4hh + i / 4) (and two rows further),
    // column col0 + 16g + 4(i & 3).  Per lane only a base address varies; the
    // stage, chunk, column block and second read are immediate offsets.
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    typedef __attribute__((address_space(3))) char lds_char;
    const int ri = lane & 15, rg = (lane >> 4) & 1;
    const int rrow = 4 * (ri >> 2) + hh, rcol = 16 * rg + 4 * (ri & 3);
    lds_char* const kb = (lds_char*)(uintptr_t)(uint32_t)(uintptr_t)(smem + rrow * RS + rcol);
    lds_char* const sb = (lds_char*)(uintptr_t)(uint32_t)(uintptr_t)(smem + KTILE + rrow * RQ + wave * 32 + rcol);
    auto tr_pair = [](lds_char* at, int rs_bytes) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)at);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(at + 2 * rs_bytes));
        uint4 u;
        u.x = __builtin_bit_cast(uint2, lo).x;
        u.y = __builtin_bit_cast(uint2, lo).y;
        u.z = __builtin_bit_cast(uint2, hi).x;
        u.w = __builtin_bit_cast(uint2, hi).y;
        return u;
    };
    // dQ^T (rows e, columns queries) += K^T dS^T over the block's 4 key chunks
    auto products = [&](auto stage_c) {
        constexpr int so = decltype(stage_c)::value * STAGE * 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint4 a[NDB];
            const uint4 bop = tr_pair(sb + so + 16 * c * RQ * 2, RQ * 2);
#pragma unroll
            for (int db = 0; db < NDB; ++db) a[db] = tr_pair(kb + so + (16 * c * RS + 32 * db) * 2, RS * 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = Tr::mfma32(as_vec8<Tr>(a[db]), as_vec8<Tr>(bop), acc[db]);
        }
    };
    // Block t sits in stage t & 1; registers ta hold even blocks, tb odd ones.
    // Each step issues the loads of block t + 2 before its products and stores
    // block t + 1 (loaded a step earlier) after them; a stage is rewritten only
    // after the barrier that ends the step which read it.
    Tile ta, tb;
    load_tile(0, ta);
    load_tile(1, tb);
    store_tile(0, ta);
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        load_tile(t + 2, ta);
        products(std::integral_constant<int, 0>{});
        store_tile(1, tb);
        __syncthreads();
        if (t + 1 >= ntiles) break;
        load_tile(t + 3, tb);
        products(std::integral_constant<int, 1>{});
        store_tile(0, ta);
        __syncthreads();
    }

    // dQ = scale * dQ^T, rounded to nearest-even; lane: query lrow, e = 32db + 8g + 4hh + 0..3
    const int lrow = wave * 32 + lq;
    const int dq_rs = (int)(p.dq_sr * 2);
    const auto ors = make_rsrc((uint16_t*)p.dq + (int64_t)b * p.dq_sb + h * p.dq_sh + (int64_t)q0 * p.dq_sr,
                               (qrows - 1) * dq_rs + D * 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + g * 8 + hh * 4;
            uint2 st;
            st.x = Tr::pack2(acc[db][4 * g + 0] * p.scale, acc[db][4 * g + 1] * p.scale);
            st.y = Tr::pack2(acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale);
            buf_store8(st, ors, lrow * dq_rs + d * 2);
        }
}

// ---------------------------------------------------------------- dK, dV

// x += sum over kk of A_kk B_kk, with A_kk the 16-byte LDS read at row + 16 kk
// (16-bit words) and B_kk = b[kk]: a chain of products into one accumulator.
// BATCH: all reads are issued before the first product, which then waits for
// the first read only (otherwise the compiler may wait for each read in turn).
template <typename Tr, int N, int RS, bool BATCH>
__device__ __forceinline__ void chain_product(const uint16_t* row, const uint4* b, f32x16_t& x) {
    if constexpr (BATCH) {
        uint4 a[N];
#pragma unroll
        for (int kk = 0; kk < N; ++kk) a[kk] = *(const uint4*)(row + kk * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < N; ++kk) x = Tr::mfma32(as_vec8<Tr>(a[kk]), as_vec8<Tr>(b[kk]), x);
    } else {
#pragma unroll
        for (int kk = 0; kk < N; ++kk) x = Tr::mfma32(as_vec8<Tr>(*(const uint4*)(row + kk * 16)), as_vec8<Tr>(b[kk]), x);
    }
}

// Eight wavefronts per 128 keys, two roles over the same 32-key slices:
// wavefronts 0-3 own dV (S, P, dV^T += dO^T P), wavefronts 4-7 own dK (dP,
// dS, dK^T += Q^T dS); wavefronts w and w + 4 share a SIMD.  Each step (64
// queries) runs in two phases split by barriers, the dK role one step behind:
// in phase A the dV role forms P of step t (the S product and its
// exponentials; P written to LDS in fp32 and kept packed for the dV product)
// while the dK role forms dS of step t - 1 and its dK product; in phase B the
// dV role runs the dV product and the dK role dP of step t.  Both roles then
// carry one product chain plus like vector work in phase A and one product
// chain in phase B, so neither waits long at the barriers (with dS and the dK
// product in the phase of the dV product, each role used to wait ~18% of a
// step for the other).
template <typename Tr, int D, bool CAUSAL, int MASK = MASK_NONE, bool VARLEN = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p) {
    static_assert(!(VARLEN && MASK != MASK_NONE), "packed batches take no mask");
    constexpr int BK = 128, BN = 64;     // keys per workgroup, queries per step
    constexpr int NT = 512;
    constexpr int RS = D + 8;
    constexpr int TILE = BN * RS;
    constexpr int STAGE = 2 * TILE + 2 * BN * 2;  // Q, dO, then lse*log2e and D (fp32, natural order)
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int NCH = BN * D / 8;
    constexpr int NCH_T = (NCH + NT - 1) / NT;
    constexpr int PX = 2 * 4 * 2 * 64 * 16;       // P exchange: 2 step parities x 4 key slices x 2 query halves x 64 lanes x 16
    // operand reads of a product chain issued together
    constexpr bool kBatchReads = true;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) float pex[PX];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it stay scalar
    // role 0 forms P and accumulates dV; role 1 forms dP and dS and accumulates dK.
    // Waves kw and kw + 4 (one of each role, same keys) share a SIMD.
    const int role = __builtin_amdgcn_readfirstlane(wave >> 2);
    const int kw = wave & 3;
    const int lq = lane & 31, hh = lane >> 5;
    const int nbh = p.Hkv * p.B;
    const int kt = (int)(blockIdx.x / nbh);   // lowest key tiles (most causal work) first
    const int bkv = (int)(blockIdx.x % nbh);
    const int kvh = bkv % p.Hkv, b = bkv / p.Hkv;
    int Lb = p.L, Sb = p.S;
    int64_t qa = 0, kc = 0;  // packed batches: first token of segment b's rows and keys
    if constexpr (VARLEN) bwd_segment(p, b, qa, Lb, kc, Sb);
    const int64_t q_b = VARLEN ? qa * p.q_sr : b * p.q_sb, do_b = VARLEN ? qa * p.do_sr : b * p.do_sb;
    const int64_t k_b = VARLEN ? kc * p.k_sr : b * p.k_sb, v_b = VARLEN ? kc * p.v_sr : b * p.v_sb;
    const int k0 = kt * BK;
    if (k0 >= Sb) return;
    const int krows = min(BK, Sb - k0);
    const int wkey0 = k0 + kw * 32;            // first key of this wavefront
    const int my_key = wkey0 + lq;
    const bool wave_has_keys = kw * 32 < krows;

    // K^T (role 0) or V^T (role 1) operand (lane: key lq, elements 16kk + 8hh .. +7)
    const int k_rs = (int)(p.k_sr * 2), v_rs = (int)(p.v_sr * 2);
    const auto krs = make_rsrc((const uint16_t*)p.k + k_b + kvh * p.k_sh + (int64_t)k0 * p.k_sr,
                               (krows - 1) * k_rs + D * 2);
    const auto vrs = make_rsrc((const uint16_t*)p.v + v_b + kvh * p.v_sh + (int64_t)k0 * p.v_sr,
                               (krows - 1) * v_rs + D * 2);
    const int lkey = kw * 32 + lq;
    uint4 kvreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
        kvreg[kk] = role == 0 ? buf_load16(krs, lkey * k_rs + (kk * 16 + hh * 8) * 2)
                              : buf_load16(vrs, lkey * v_rs + (kk * 16 + hh * 8) * 2);
    const float c2 = p.scale * kLog2e;
    wait_vmem_all();  // as in the dQ kernel: no wait for these inside the loop

    f32x16_t acc[NDB];  // dV^T (role 0) or dK^T (role 1): rows e, columns keys
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

    // query blocks this workgroup visits: causal keeps query i >= key j
    const int qb0 = CAUSAL ? k0 / BN : 0;
    const int nqb = (Lb + BN - 1) / BN;
    const int nsteps = p.group * max(0, nqb - qb0);  // (query head, query block) pairs

    const int q_rs = (int)(p.q_sr * 2), do_rs = (int)(p.do_sr * 2);
    uint4 qbuf[NCH_T], gbuf[NCH_T];
    float lbuf = 0.f, dbuf = 0.f;
    auto step_coords = [&](int st, int& h, int& qrow0) {
        h = kvh * p.group + st / max(1, nqb - qb0);
        qrow0 = (qb0 + st % max(1, nqb - qb0)) * BN;
    };
    auto load_tile = [&](int st) {
        int h, qrow0;
        step_coords(st, h, qrow0);
        const int rows = min(BN, Lb - qrow0);
        const auto qr = make_rsrc((const uint16_t*)p.q + q_b + h * p.q_sh + (int64_t)qrow0 * p.q_sr,
                                  (rows - 1) * q_rs + D * 2);
        const auto gr = make_rsrc((const uint16_t*)p.dout + do_b + h * p.do_sh + (int64_t)qrow0 * p.do_sr,
                                  (rows - 1) * do_rs + D * 2);
#pragma unroll
        for (int i = 0; i < NCH_T; ++i) {
            const int ch = tid + NT * i, r = ch / (D / 8), col = (ch % (D / 8)) * 8;
            if (NCH % NT == 0 || ch < NCH) {
                qbuf[i] = buf_load16(qr, r * q_rs + col * 2);
                gbuf[i] = buf_load16(gr, r * do_rs + col * 2);
            }
        }
        if (tid < BN) {
            // raw values (range-checked loads read 0 past the last row); scaled
            // when stored, so that nothing here waits for the loads
            const int64_t rowid = VARLEN ? (int64_t)h * p.total_q + qa : ((int64_t)b * p.Hq + h) * p.L;
            const int64_t lse_b = VARLEN ? h * p.lse_sh + qa : b * p.lse_sb + h * p.lse_sh;
            const auto lr = make_rsrc(p.lse + lse_b + qrow0, rows * 4);
            const auto dr = make_rsrc(p.dsum + rowid + qrow0, rows * 4);
            lbuf = __uint_as_float(buf_load4(lr, tid * 4));
            dbuf = __uint_as_float(buf_load4(dr, tid * 4));
        }
    };
    auto store_tile = [&](int stage) {
        uint16_t* Qs = smem + stage * STAGE;
        uint16_t* Gs = Qs + TILE;
        float* Ls = (float*)(Gs + TILE);
#pragma unroll
        for (int i = 0; i < NCH_T; ++i) {
            const int ch = tid + NT * i, r = ch / (D / 8), col = (ch % (D / 8)) * 8;
            if (NCH % NT == 0 || ch < NCH) {
                *(uint4*)(Qs + bwd_pos(r) * RS + col) = qbuf[i];
                *(uint4*)(Gs + bwd_pos(r) * RS + col) = gbuf[i];
            }
        }
        if (tid < BN) {
            // a masked row with no kept key (lse -inf) has P = 0: exp2(-inf - 0)
            Ls[tid] = (MASK != MASK_NONE && lbuf == kNegInf) ? 0.f : lbuf * kLog2e;
            Ls[BN + tid] = dbuf;
        }
    };

    // this wave's P exchange area for the steps of parity x, query half qb:
    // float4 j of lane l at (j * 64 + l) * 4
    auto px_of = [&](int x, int qb) { return pex + x * (PX / 2) + kw * (2 * 64 * 16) + qb * (64 * 16); };
    // causal: the wave's keys need queries >= wkey0
    auto active_at = [&](int qrow0) { return wave_has_keys && (!CAUSAL || qrow0 + BN - 1 >= wkey0); };
    // acc += X^T op over the two 16-query chunks of query half qb: X = dO (role
    // 0, op = P) or Q (role 1, op = dS), read transposed from the stage at Xs
    // dS^T of this workgroup's keys, when the call keeps it (batched calls):
    // lane (key lkey, queries qrow0 + 32qb + 16c + 8hh + 0..7) stores 16 bytes
    // per chunk c into the 128-query panel of qrow0; keys past the last, and
    // every store when keep is false, are dropped by the buffer range
    auto store_ds = [&](bool keep, int h, int qrow0, int qb, const uint4* op) {
        const auto r = make_rsrc(keep ? p.ds + (((int64_t)b * p.Hq + h) * p.ds_lp + (qrow0 & ~127)) * p.S + (int64_t)k0 * 128
                                      : p.ds,
                                 keep ? krows * 256 : 0);
#pragma unroll
        for (int c = 0; c < 2; ++c) buf_store16_nt(op[c], r, (lkey * 128 + (qrow0 & 127) + 32 * qb + 16 * c + 8 * hh) * 2);
    };
    auto transposed_products = [&](const uint16_t* Xs, int qb, const uint4* op) {
        uint4 xa[2][NDB];   // all reads first: the products wait for the first only
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db) xa[c][db] = read_tr<RS>(Xs, qb * 2 + c, db * 32, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = Tr::mfma32(as_vec8<Tr>(xa[c][db]), as_vec8<Tr>(op[c]), acc[db]);
    };

    if (nsteps > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    // Iteration it: phase A, role 0 forms P of step it, role 1 dS and dK of step
    // it - 1; barrier; phase B, role 0 the dV product of step it, role 1 dP of
    // step it; barrier.  Both phases then carry like work on the two roles.
    // The two roles run the same sequence of barriers in separate loops (their
    // values then do not compete for registers).
    if (role == 0) {
        uint4 pw[2][2];   // P of the current step, packed as B operands
        for (int it = 0; it <= nsteps; ++it) {
            if (it + 1 < nsteps) load_tile(it + 1);
            // phase A: P of step it
            if (it < nsteps) {
                int h, qrow0;
                step_coords(it, h, qrow0);
                const uint16_t* Qs = smem + (it & 1) * STAGE;
                const float* Ls = (const float*)(Qs + 2 * TILE);
                if (active_at(qrow0)) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        // mask values of this lane's key for the 16 queries of register r
                        // (query 32qb + 16(r/8) + 8hh + r%8 of the block), loaded before the products
                        float mb[16];
                        uint32_t mk = ~0u;
                        if constexpr (MASK != MASK_NONE) {
                            constexpr int MES = MASK == MASK_FLOAT ? 4 : 1;
                            const int qf = qrow0 + qb * 32, nq = Lb - qf;
                            const auto mr = make_rsrc((const char*)p.mask + ((int64_t)b * p.m_sb + (int64_t)h * p.m_sh +
                                                                             (int64_t)qf * p.m_sr + wkey0) * MES,
                                                      nq > 0 ? ((nq - 1) * (int)p.m_sr + (Sb - wkey0)) * MES : 0);
                            mk = 0;
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int off = ((16 * (r >> 3) + 8 * hh + (r & 7)) * (int)p.m_sr + lq) * MES;
                                if constexpr (MASK == MASK_FLOAT)
                                    mb[r] = __uint_as_float(buf_load4(mr, off));
                                else
                                    mk |= (buf_load1(mr, off) != 0 ? 1u : 0u) << r;
                            }
                        }
                        f32x16_t sc = f32x16_t{};
                        chain_product<Tr, NKK, RS, kBatchReads>(Qs + bwd_rowpos(qb * 32 + lq) * RS + hh * 8, kvreg, sc);
                        // register r: query qrow0 + 32qb + 16(r/8) + 8hh + r%8, key my_key
                        const int qbase = qb * 32 + 8 * hh;
                        const bool edge = (qrow0 + BN > Lb) || (CAUSAL && qrow0 < wkey0 + 31);
                        float w[16];
                        // two copies, with and without the edge test (see the dQ kernel)
                        auto weights = [&](auto edge_c) {
#pragma unroll
                            for (int half = 0; half < 2; ++half) {
                                const float4 la = *(const float4*)(Ls + qbase + 16 * half);
                                const float4 lb = *(const float4*)(Ls + qbase + 16 * half + 4);
                                const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
#pragma unroll
                                for (int j = 0; j < 8; ++j) {
                                    const int r = 8 * half + j;
                                    float e;
                                    if constexpr (MASK == MASK_FLOAT)
                                        e = fast_exp2(fmaf(fmaf(sc[r], p.scale, mb[r]), kLog2e, -lv[j]));
                                    else
                                        e = fast_exp2(fmaf(sc[r], c2, -lv[j]));
                                    if constexpr (MASK == MASK_BOOL) e = ((mk >> r) & 1u) ? e : 0.f;
                                    if constexpr (decltype(edge_c)::value) {
                                        const int qi = qrow0 + qbase + 16 * half + j;
                                        const bool keep = qi < Lb && (!CAUSAL || qi >= my_key);
                                        e = keep ? e : 0.f;
                                    }
                                    w[r] = e;
                                }
                            }
                        };
                        if (edge)
                            weights(std::true_type{});
                        else
                            weights(std::false_type{});
                        float* pq = px_of(it & 1, qb);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            *(float4*)(pq + (j * 64 + lane) * 4) = make_float4(w[4 * j], w[4 * j + 1], w[4 * j + 2],
                                                                               w[4 * j + 3]);
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            pw[qb][c].x = Tr::pack2(w[c * 8 + 0], w[c * 8 + 1]);
                            pw[qb][c].y = Tr::pack2(w[c * 8 + 2], w[c * 8 + 3]);
                            pw[qb][c].z = Tr::pack2(w[c * 8 + 4], w[c * 8 + 5]);
                            pw[qb][c].w = Tr::pack2(w[c * 8 + 6], w[c * 8 + 7]);
                        }
                    }
                }
            }
            __syncthreads();   // P of step it is in the exchange area
            // phase B: dV^T += dO^T P of step it
            if (it < nsteps) {
                int h, qrow0;
                step_coords(it, h, qrow0);
                (void)h;
                const uint16_t* Gs = smem + (it & 1) * STAGE + TILE;
                if (active_at(qrow0)) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) transposed_products(Gs, qb, pw[qb]);
                }
            }
            if (it + 1 < nsteps) store_tile((it + 1) & 1);
            __syncthreads();
        }
    } else {
        f32x16_t dp[2];   // dP of the previous step, kept for its dS
        for (int it = 0; it <= nsteps; ++it) {
            if (it + 1 < nsteps) load_tile(it + 1);
            // phase A: dS and dK of step it - 1
            {
                // dS = P (dP - D) of step it - 1 (its P in the exchange area since the
                // previous iteration, its Q, D still in their stage), dK^T += Q^T dS.
                // The dS^T stores are issued on every iteration (an empty range when
                // nothing is kept, zeros for a slice with no kept key), so the number
                // of memory operations after the next tile's loads is the same on
                // every path and the wait for those loads leaves the stores in flight.
                const int st = it > 0 ? it - 1 : 0;
                int h, qrow0;
                step_coords(st, h, qrow0);
                const uint16_t* Qs = smem + (st & 1) * STAGE;
                const float* Ls = (const float*)(Qs + 2 * TILE);
                const bool act = it > 0 && active_at(qrow0);
                const bool keep_ds = !VARLEN && it > 0 && p.ds != nullptr;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    uint4 op[2] = {zero4(), zero4()};
                    if (act) {
                        const float* pq = px_of(st & 1, qb);
                        const int qbase = qb * 32 + 8 * hh;
                        float w[16];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float4 e4 = *(const float4*)(pq + (j * 64 + lane) * 4);
                            w[4 * j] = e4.x; w[4 * j + 1] = e4.y; w[4 * j + 2] = e4.z; w[4 * j + 3] = e4.w;
                        }
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const float4 da = *(const float4*)(Ls + BN + qbase + 16 * half);
                            const float4 db4 = *(const float4*)(Ls + BN + qbase + 16 * half + 4);
                            const float dv8[8] = {da.x, da.y, da.z, da.w, db4.x, db4.y, db4.z, db4.w};
#pragma unroll
                            for (int j = 0; j < 8; ++j) w[8 * half + j] = w[8 * half + j] * (dp[qb][8 * half + j] - dv8[j]);
                        }
#pragma unroll
                        for (int c = 0; c < 2; ++c) {
                            op[c].x = Tr::pack2(w[c * 8 + 0], w[c * 8 + 1]);
                            op[c].y = Tr::pack2(w[c * 8 + 2], w[c * 8 + 3]);
                            op[c].z = Tr::pack2(w[c * 8 + 4], w[c * 8 + 5]);
                            op[c].w = Tr::pack2(w[c * 8 + 6], w[c * 8 + 7]);
                        }
                    }
                    if constexpr (!VARLEN) store_ds(keep_ds, h, qrow0, qb, op);
                    if (act) transposed_products(Qs, qb, op);
                }
            }
            __syncthreads();   // step it - 1's stage is no longer read
            // phase B: dP = dO V^T of step it
            if (it < nsteps) {
                int h, qrow0;
                step_coords(it, h, qrow0);
                (void)h;
                const uint16_t* Gs = smem + (it & 1) * STAGE + TILE;
                if (active_at(qrow0)) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        dp[qb] = f32x16_t{};
                        chain_product<Tr, NKK, RS, kBatchReads>(Gs + bwd_rowpos(qb * 32 + lq) * RS + hh * 8,
                                                                kvreg, dp[qb]);
                    }
                }
            }
            if (it + 1 < nsteps) store_tile((it + 1) & 1);
            __syncthreads();
        }
    }

    // dV = dV^T or dK = scale * dK^T, rounded to nearest-even; lane: key lkey, e = 32db + 8g + 4hh + 0..3
    const float f = role == 1 ? p.scale : 1.f;
    const int o_rs = (int)((role == 1 ? p.dk_sr : p.dv_sr) * 2);
    void* obase = role == 1 ? p.dk : p.dv;
    const int64_t o_sb = role == 1 ? p.dk_sb : p.dv_sb, o_sh = role == 1 ? p.dk_sh : p.dv_sh;
    const int64_t o_sr = role == 1 ? p.dk_sr : p.dv_sr;
    const auto ors = make_rsrc((uint16_t*)obase + (VARLEN ? kc * o_sr : b * o_sb) + kvh * o_sh + (int64_t)k0 * o_sr,
                               (krows - 1) * o_rs + D * 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + g * 8 + hh * 4;
            uint2 st;
            st.x = Tr::pack2(acc[db][4 * g + 0] * f, acc[db][4 * g + 1] * f);
            st.y = Tr::pack2(acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f);
            buf_store8(st, ors, lkey * o_rs + d * 2);
        }
}

template <typename Tr, int D, bool CAUSAL, int MASK, bool VARLEN>
void launch_bwd_grads(const BwdParams& p, hipStream_t s) {
    const unsigned gq = (unsigned)p.n_qtiles * p.Hq * p.B;
    const unsigned gk = (unsigned)p.n_ktiles * p.Hkv * p.B;
    if (!VARLEN && p.ds) {
        // D, then dK/dV (storing dS^T), then dQ from dS^T
        if ((int64_t)p.B * p.Hq * p.L > 0)
            hipLaunchKernelGGL((bwd_dsum_kernel<Tr, D>), dim3(gq), dim3(256), 0, s, p);
        if ((int64_t)p.S * p.Hkv * p.B > 0)
            hipLaunchKernelGGL((bwd_dkdv_kernel<Tr, D, CAUSAL, MASK, VARLEN>), dim3(gk), dim3(512), 0, s, p);
        if ((int64_t)p.B * p.Hq * p.L > 0)
            hipLaunchKernelGGL((bwd_dq_ds_kernel<Tr, D, CAUSAL>), dim3(gq), dim3(256), 0, s, p);
        return;
    }
    if ((int64_t)p.B * p.Hq * p.L > 0)
        hipLaunchKernelGGL((bwd_dq_kernel<Tr, D, CAUSAL, MASK, VARLEN>), dim3(gq), dim3(256), 0, s, p);
    if ((int64_t)p.S * p.Hkv * p.B > 0)
        hipLaunchKernelGGL((bwd_dkdv_kernel<Tr, D, CAUSAL, MASK, VARLEN>), dim3(gk), dim3(512), 0, s, p);
}

template <typename Tr, int D, int MASK, bool VARLEN = false>
void launch_bwd_m(const BwdParams& p, bool causal, hipStream_t s) {
    if (causal)
        launch_bwd_grads<Tr, D, true, MASK, VARLEN>(p, s);
    else
        launch_bwd_grads<Tr, D, false, MASK, VARLEN>(p, s);
}

template <typename Tr, int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, int mask, bool varlen, hipStream_t s) {
    if (varlen) {
        if (mask != MASK_NONE) return hipErrorInvalidValue;
        launch_bwd_m<Tr, D, MASK_NONE, true>(p, causal, s);
        return hipGetLastError();
    }
    switch (mask) {
        case MASK_NONE: launch_bwd_m<Tr, D, MASK_NONE>(p, causal, s); break;
        case MASK_FLOAT: launch_bwd_m<Tr, D, MASK_FLOAT>(p, causal, s); break;
        case MASK_BOOL: launch_bwd_m<Tr, D, MASK_BOOL>(p, causal, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename Tr>
hipError_t launch_bwd_t(const BwdParams& p, int D, bool causal, int mask, bool varlen, hipStream_t s) {
    switch (D) {
        case 64: return launch_bwd_d<Tr, 64>(p, causal, mask, varlen, s);
        case 96: return launch_bwd_d<Tr, 96>(p, causal, mask, varlen, s);
        case 128: return launch_bwd_d<Tr, 128>(p, causal, mask, varlen, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward(const BwdParams& p, int D, bool causal, int mask, bool varlen, hipStream_t stream) {
    return p.elem == ELEM_BF16 ? launch_bwd_t<BF16>(p, D, causal, mask, varlen, stream)
                               : launch_bwd_t<F16>(p, D, causal, mask, varlen, stream);
}

}  // namespace sdpa

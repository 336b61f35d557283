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
// Two kernels:
//   bwd_dq_kernel     one workgroup per 128 query rows (4 wavefronts x 32);
//                     first D_i = dO_i . O_i in fp32 from the dO rows it holds
//                     and the O rows in the same layout (written to the
//                     workspace for the second kernel, which runs after it);
//                     for each 64-key block, S^T = K Q^T and dP^T = V dO^T on
//                     the matrix cores (the transposed score layout of the
//                     forward kernels, one query per lane), P^T and dS^T in
//                     registers, then dQ^T += K^T dS^T with dS^T as the B
//                     operand straight from the score registers and K^T read
//                     from LDS with the transposing ds_read_b64_tr_b16.
//   bwd_dkdv_kernel   one workgroup per 128 keys, over the query heads of the
//                     key/value head and their 64-row query blocks, with two
//                     roles per 32-key slice: one wavefront computes S = Q K^T
//                     and dP = dO V^T (one key per lane) and dK^T += Q^T dS,
//                     another S and dV^T += dO^T P; P and dS are B operands
//                     from the score registers, dO^T and Q^T are read
//                     transposed from LDS.
// No atomics: each gradient element has one owner.  The price is that S is
// computed three times and dP twice, 8 matrix products per kept (query, key)
// pair and head dimension instead of the 5 of one shared pass; in exchange
// every wavefront fits in 256 registers (two per SIMD).
//
// Optional masks, as in the forward: a float32 bias enters the logit as
// scale * s + bias, a bool mask sets P = 0 on the keys it drops; the dQ kernel
// reads its row's mask in 8-key runs, the dK/dV kernel down its key's column.
// A row whose forward kept no key (lse -inf) is read with lse 0, so all its
// weights are exp(-inf) = 0 and it contributes nothing.  Packed
// variable-length batches (block-diagonal mask) take each segment's first
// token and lengths from cu_seqlens and address rows by token.
//
// LDS tiles are row-major with 8 elements of padding per row (16-byte row
// reads conflict-free).  Rows are stored at position swap23(r) within each
// 32-row group (bits 2 and 3 of the row index swapped): then register r of
// lane l of a 32x32 product tile holds row 16(r/8) + 8(l/32) + r%8 of its
// group, which is exactly the k-slot order of a B operand, and each group of
// 4 consecutive natural rows stays at 4 consecutive positions, as the
// transposing reads need.
#include "attn_common.h"
#include "device_utils.h"

namespace sdpa {

namespace {

__device__ __forceinline__ int bwd_swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int bwd_pos(int r) { return (r & ~31) | bwd_swap23(r & 31); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// A operand X^T (32 columns of X as rows, 16 rows of X as k-slots) of one
// 16-row chunk c of a row-major tile X[pos][RS] (16-bit words): lane l gets
// column col0 + (l & 31) and natural rows 16c + 8(l/32) + 0..7, in two
// transposing reads of 4 rows each.
template <int RS>
__device__ __forceinline__ uint4 read_tr(const uint16_t* tile, int c, int col0, int lane) {
    const int i = lane & 15, g = (lane >> 4) & 1, hh = lane >> 5;
    const int col = col0 + 16 * g + 4 * (i & 3);
    const uint16_t* a0 = tile + (16 * c + 4 * hh + (i >> 2)) * RS + col;
    const uint16_t* a1 = tile + (16 * c + 8 + 4 * hh + (i >> 2)) * RS + col;
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
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint4 ka = *(const uint4*)(Ks + (kb * 32 + lq) * RS + kk * 16 + hh * 8);
                    const uint4 va = *(const uint4*)(Vs + (kb * 32 + lq) * RS + kk * 16 + hh * 8);
                    s[kb] = Tr::mfma32(as_vec8<Tr>(ka), as_vec8<Tr>(qreg[kk]), s[kb]);
                    dp[kb] = Tr::mfma32(as_vec8<Tr>(va), as_vec8<Tr>(dreg[kk]), dp[kb]);
                }
            // register r of block kb: key key0 + 32kb + 16(r/8) + 8hh + r%8, query my_row
            const bool edge = (key0 + BN > Sb) || (CAUSAL && key0 + BN - 1 > q0 + wrow0);
            int lim = Sb - (key0 + hh * 8);
            if (CAUSAL) lim = min(lim, my_row + 1 - (key0 + hh * 8));
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
                    if (edge) pv = (kb * 32 + (r >> 3) * 16 + (r & 7) < lim) ? pv : 0.f;
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
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint4 a = read_tr<RS>(Ks, c, db * 32, lane);
                    acc[db] = Tr::mfma32(as_vec8<Tr>(a), as_vec8<Tr>(pb[c]), acc[db]);
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

// ---------------------------------------------------------------- dK, dV

// Eight wavefronts per 128 keys, two roles over the same 32-key slices:
// wavefronts 0-3 own dK (S, dP, dS, dK^T += Q^T dS), wavefronts 4-7 own dV
// (S, P, dV^T += dO^T P).  Each role fits two wavefronts per SIMD; S is
// computed by both roles.
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
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int role = __builtin_amdgcn_readfirstlane(wave >> 2);  // 0: dK, 1: dV
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

    // K^T (and for dK, V^T) operands (lane: key lq, elements 16kk + 8hh .. +7)
    const int k_rs = (int)(p.k_sr * 2), v_rs = (int)(p.v_sr * 2);
    const auto krs = make_rsrc((const uint16_t*)p.k + k_b + kvh * p.k_sh + (int64_t)k0 * p.k_sr,
                               (krows - 1) * k_rs + D * 2);
    const auto vrs = make_rsrc((const uint16_t*)p.v + v_b + kvh * p.v_sh + (int64_t)k0 * p.v_sr,
                               (krows - 1) * v_rs + D * 2);
    const int lkey = kw * 32 + lq;
    uint4 kreg[NKK], vreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        kreg[kk] = buf_load16(krs, lkey * k_rs + (kk * 16 + hh * 8) * 2);
        vreg[kk] = role == 0 ? buf_load16(vrs, lkey * v_rs + (kk * 16 + hh * 8) * 2) : zero4();
    }
    const float c2 = p.scale * kLog2e;
    wait_vmem_all();  // as in the dQ kernel: no wait for these inside the loop

    f32x16_t acc[NDB];  // dK^T (role 0) or dV^T (role 1): rows e, columns keys
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

    if (nsteps > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        if (st + 1 < nsteps) load_tile(st + 1);
        int h, qrow0;
        step_coords(st, h, qrow0);
        const uint16_t* Qs = smem + (st & 1) * STAGE;
        const uint16_t* Gs = Qs + TILE;
        const float* Ls = (const float*)(Gs + TILE);
        // causal: the wave's keys need queries >= wkey0
        const bool active = wave_has_keys && (!CAUSAL || qrow0 + BN - 1 >= wkey0);
        if (active) {
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
                f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const uint4 qa = *(const uint4*)(Qs + (qb * 32 + lq) * RS + kk * 16 + hh * 8);
                    s = Tr::mfma32(as_vec8<Tr>(qa), as_vec8<Tr>(kreg[kk]), s);
                }
                if (role == 0) {
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const uint4 ga = *(const uint4*)(Gs + (qb * 32 + lq) * RS + kk * 16 + hh * 8);
                        dp = Tr::mfma32(as_vec8<Tr>(ga), as_vec8<Tr>(vreg[kk]), dp);
                    }
                }
                // register r: query qrow0 + 32qb + 16(r/8) + 8hh + r%8, key my_key
                const int qbase = qb * 32 + 8 * hh;
                const bool edge = (qrow0 + BN > Lb) || (CAUSAL && qrow0 < wkey0 + 31);
                float w[16];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float4 la = *(const float4*)(Ls + qbase + 16 * half);
                    const float4 lb = *(const float4*)(Ls + qbase + 16 * half + 4);
                    const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
                    float dv8[8];
                    if (role == 0) {
                        const float4 da = *(const float4*)(Ls + BN + qbase + 16 * half);
                        const float4 db4 = *(const float4*)(Ls + BN + qbase + 16 * half + 4);
                        dv8[0] = da.x; dv8[1] = da.y; dv8[2] = da.z; dv8[3] = da.w;
                        dv8[4] = db4.x; dv8[5] = db4.y; dv8[6] = db4.z; dv8[7] = db4.w;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = 8 * half + j;
                        float e;
                        if constexpr (MASK == MASK_FLOAT)
                            e = fast_exp2(fmaf(fmaf(s[r], p.scale, mb[r]), kLog2e, -lv[j]));
                        else
                            e = fast_exp2(fmaf(s[r], c2, -lv[j]));
                        if constexpr (MASK == MASK_BOOL) e = ((mk >> r) & 1u) ? e : 0.f;
                        if (edge) {
                            const int qi = qrow0 + qbase + 16 * half + j;
                            const bool keep = qi < Lb && (!CAUSAL || qi >= my_key);
                            e = keep ? e : 0.f;
                        }
                        w[r] = role == 0 ? e * (dp[r] - dv8[j]) : e;  // dS or P
                    }
                }
                uint4 pw[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    pw[c].x = Tr::pack2(w[c * 8 + 0], w[c * 8 + 1]);
                    pw[c].y = Tr::pack2(w[c * 8 + 2], w[c * 8 + 3]);
                    pw[c].z = Tr::pack2(w[c * 8 + 4], w[c * 8 + 5]);
                    pw[c].w = Tr::pack2(w[c * 8 + 6], w[c * 8 + 7]);
                }
                // dK^T += Q^T dS (role 0) or dV^T += dO^T P (role 1) over two 16-query chunks
                const uint16_t* Xs = role == 0 ? Qs : Gs;
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const uint4 xa = read_tr<RS>(Xs, qb * 2 + c, db * 32, lane);
                        acc[db] = Tr::mfma32(as_vec8<Tr>(xa), as_vec8<Tr>(pw[c]), acc[db]);
                    }
            }
        }
        if (st + 1 < nsteps) store_tile((st + 1) & 1);
        __syncthreads();
    }

    // dK = scale * dK^T or dV = dV^T, rounded to nearest-even; lane: key lkey, e = 32db + 8g + 4hh + 0..3
    const float f = role == 0 ? p.scale : 1.f;
    const int o_rs = (int)((role == 0 ? p.dk_sr : p.dv_sr) * 2);
    void* obase = role == 0 ? p.dk : p.dv;
    const int64_t o_sb = role == 0 ? p.dk_sb : p.dv_sb, o_sh = role == 0 ? p.dk_sh : p.dv_sh;
    const int64_t o_sr = role == 0 ? p.dk_sr : p.dv_sr;
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
    if ((int64_t)p.B * p.Hq * p.L > 0) {
        const unsigned g = (unsigned)p.n_qtiles * p.Hq * p.B;
        hipLaunchKernelGGL((bwd_dq_kernel<Tr, D, CAUSAL, MASK, VARLEN>), dim3(g), dim3(256), 0, s, p);
    }
    if ((int64_t)p.S * p.Hkv * p.B > 0) {
        const unsigned g = (unsigned)p.n_ktiles * p.Hkv * p.B;
        hipLaunchKernelGGL((bwd_dkdv_kernel<Tr, D, CAUSAL, MASK, VARLEN>), dim3(g), dim3(512), 0, s, p);
    }
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

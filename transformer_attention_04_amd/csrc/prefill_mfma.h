// Single-pass attention forward for bf16 / fp16 inputs on gfx950 matrix cores.
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
//    wavefront owns 32 rows.  Keys advance 64 per step through a
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
//  * V^T rows are XOR-swizzled in 16-byte chunks by (row / 8) % 8 so that the
//    transposing writes and the 16-byte MFMA operand reads avoid LDS bank
//    conflicts.
//  * Causal: key blocks wholly above the diagonal are never loaded; wavefronts
//    whose rows all precede a block skip its products; masking by index runs
//    only on edge blocks.  Workgroups are dispatched heaviest query block first.
//  * Special rows: a row with no kept key keeps running max -inf, uses a zero
//    shift, and ends with output 0 and lse -inf; a NaN score makes exp NaN and
//    the row NaN.
#pragma once

#include "attn_common.h"
#include "device_utils.h"

namespace sdpa {

// Swap bits 2 and 3 of a key index within its 32-key block.
__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <typename Tr, int D, bool CAUSAL, int MASK, bool VARLEN>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(AttnParams p) {
    constexpr int BM = kPrefillBlockM;
    constexpr int BN = 64;
    constexpr int KS = D + 8;      // LDS row stride of the K tile, in 16-bit words
    constexpr int VS = BN + 8;     // LDS row stride of the V^T tile
    constexpr int KTILE = BN * KS;
    constexpr int VTILE = D * VS;
    constexpr int STAGE = KTILE + VTILE;
    constexpr int NKK = D / 16;    // k-steps of the score product
    constexpr int NDB = D / 32;    // 32-row blocks of O^T
    constexpr int KCH = BN * D / 8;          // 16-byte chunks of a K tile
    constexpr int KCH_T = (KCH + 255) / 256; // per thread
    constexpr int VIT = (D / 8) * (BN / 4);  // V items: 8 columns x 4 keys
    static_assert(D % 32 == 0, "head dim must be a multiple of 32");
    static_assert(VIT <= 256, "one V item per thread");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lq = lane & 31;
    const int hh = lane >> 5;

    const int nbh = p.Hq * p.B;
    const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / nbh);
    const int bh = (int)(blockIdx.x % nbh);
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int kvh = h / p.group;

    int Lb, Sb;
    int64_t qo, ko, vo, oo, lo, mo = 0;
    if (VARLEN) {
        const int64_t a = min(max((int64_t)p.cu_q[b], (int64_t)0), p.total_q);
        const int64_t e = min(max((int64_t)p.cu_q[b + 1], a), p.total_q);
        const int64_t c = min(max((int64_t)p.cu_k[b], (int64_t)0), p.total_k);
        const int64_t d = min(max((int64_t)p.cu_k[b + 1], c), p.total_k);
        Lb = (int)min(e - a, (int64_t)p.L);
        Sb = (int)(d - c);
        qo = a * p.q_sr + (int64_t)h * p.q_sh;
        ko = c * p.k_sr + (int64_t)kvh * p.k_sh;
        vo = c * p.v_sr + (int64_t)kvh * p.v_sh;
        oo = a * p.o_sr + (int64_t)h * p.o_sh;
        lo = (int64_t)h * p.lse_sh + a;
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
    const int kend = CAUSAL ? min(Sb, min(q0 + BM, Lb)) : Sb;
    const int ntiles = (kend + BN - 1) / BN;
    const int wrow0 = q0 + wave * 32;      // first row of this wavefront
    const int my_row = wrow0 + lq;         // the query this lane owns
    const bool wave_has_rows = wrow0 < Lb;

    // Q^T operand, resident for the whole loop (negated when the scale is negative).
    const uint16_t* qp = (const uint16_t*)p.q + qo;
    uint4 qreg[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        uint4 u = zero4();
        if (my_row < Lb) u = *(const uint4*)(qp + (int64_t)my_row * p.q_sr + kk * 16 + hh * 8);
        qreg[kk] = p.neg ? negate8(u) : u;
    }

    const uint16_t* kp = (const uint16_t*)p.k + ko;
    const uint16_t* vp = (const uint16_t*)p.v + vo;
    uint4 kbuf[KCH_T];
    uint4 vbuf[4];

    auto load_tile = [&](int key0) {
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i;
            kbuf[i] = zero4();
            if (c < KCH) {
                const int r = c / (D / 8), col = (c % (D / 8)) * 8;
                if (key0 + r < Sb) kbuf[i] = *(const uint4*)(kp + (int64_t)(key0 + r) * p.k_sr + col);
            }
        }
        if (tid < VIT) {
            const int dc = tid % (D / 8), kg = tid / (D / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + kg * 4 + r;
                vbuf[r] = (key < Sb) ? *(const uint4*)(vp + (int64_t)key * p.v_sr + dc * 8) : zero4();
            }
        }
    };

    auto store_tile = [&](int stage) {
        uint16_t* Ks = smem + stage * STAGE;
        uint16_t* Vt = Ks + KTILE;
#pragma unroll
        for (int i = 0; i < KCH_T; ++i) {
            const int c = tid + 256 * i;
            if (c < KCH) {
                const int r = c / (D / 8), col = (c % (D / 8)) * 8;
                const int row = (r & ~31) | swap_bits23(r & 31);
                *(uint4*)(Ks + row * KS + col) = kbuf[i];
            }
        }
        if (tid < VIT) {
            const int dc = tid % (D / 8), kg = tid / (D / 8);
            const uint32_t* w0 = (const uint32_t*)&vbuf[0];
            const uint32_t* w1 = (const uint32_t*)&vbuf[1];
            const uint32_t* w2 = (const uint32_t*)&vbuf[2];
            const uint32_t* w3 = (const uint32_t*)&vbuf[3];
            const int chunk = (kg >> 1) ^ (dc & 7);
            uint16_t* base = Vt + chunk * 8 + (kg & 1) * 4;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sh = (j & 1) * 16;
                const uint32_t e0 = (w0[j >> 1] >> sh) & 0xffffu;
                const uint32_t e1 = (w1[j >> 1] >> sh) & 0xffffu;
                const uint32_t e2 = (w2[j >> 1] >> sh) & 0xffffu;
                const uint32_t e3 = (w3[j >> 1] >> sh) & 0xffffu;
                *(uint2*)(base + (dc * 8 + j) * VS) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
            }
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    float m_run = kNegInf;  // running max: raw scores, or logits when a float mask is added
    float l_run = 0.f;      // this lane's share of the row sum

    const float* mrow_f = nullptr;
    const uint8_t* mrow_b = nullptr;
    if (MASK == MASK_FLOAT)
        mrow_f = (const float*)p.mask + mo + (int64_t)min(my_row, Lb - 1) * p.m_sr;
    if (MASK == MASK_BOOL)
        mrow_b = (const uint8_t*)p.mask + mo + (int64_t)min(my_row, Lb - 1) * p.m_sr;

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
        const bool active = wave_has_rows && (!CAUSAL || key0 <= wrow0 + 31);
        if (active) {
            f32x16_t s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16_t{};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const uint4 a = *(const uint4*)(Ks + (kb * 32 + lq) * KS + kk * 16 + hh * 8);
                    s[kb] = Tr::mfma32(as_vec8<Tr>(a), as_vec8<Tr>(qreg[kk]), s[kb]);
                }
            }
            // s[kb][8c + j] is the score of key key0 + 32kb + 16c + 8hh + j for query my_row.
            const bool edge = (key0 + BN > Sb) || (CAUSAL && key0 + BN - 1 > wrow0);
            if (MASK == MASK_FLOAT) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int base = key0 + kb * 32 + c * 16 + hh * 8;
                        float bias[8];
                        if (p.mask_vec && base + 8 <= Sb) {
                            const float4 b0 = *(const float4*)(mrow_f + base);
                            const float4 b1 = *(const float4*)(mrow_f + base + 4);
                            bias[0] = b0.x; bias[1] = b0.y; bias[2] = b0.z; bias[3] = b0.w;
                            bias[4] = b1.x; bias[5] = b1.y; bias[6] = b1.z; bias[7] = b1.w;
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j) bias[j] = (base + j < Sb) ? mrow_f[base + j] : kNegInf;
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            s[kb][c * 8 + j] = fmaf(s[kb][c * 8 + j], p.scale_abs, bias[j]);
                    }
            }
            bool keep[2][16];
            const bool any_mask = edge || MASK == MASK_BOOL;
            if (any_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int base = key0 + kb * 32 + c * 16 + hh * 8;
                        uint8_t mb[8] = {1, 1, 1, 1, 1, 1, 1, 1};
                        if (MASK == MASK_BOOL) {
                            if (p.mask_vec && base + 8 <= Sb) {
                                const uint2 u = *(const uint2*)(mrow_b + base);
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    mb[j] = (u.x >> (8 * j)) & 0xff;
                                    mb[4 + j] = (u.y >> (8 * j)) & 0xff;
                                }
                            } else {
#pragma unroll
                                for (int j = 0; j < 8; ++j) mb[j] = (base + j < Sb) ? mrow_b[base + j] : 0;
                            }
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int key = base + j;
                            bool k_ok = key < Sb && mb[j] != 0;
                            if (CAUSAL) k_ok = k_ok && key <= my_row;
                            keep[kb][c * 8 + j] = k_ok;
                            if (!k_ok) s[kb][c * 8 + j] = kNegInf;
                        }
                    }
            }
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, xor_lane(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            float alpha, tsum = 0.f;
            if (MASK == MASK_FLOAT) {
                const float shift = (m_new == kNegInf) ? 0.f : m_new;
                alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_new) * kLog2e);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = fast_exp2((s[kb][r] - shift) * kLog2e);
                        s[kb][r] = e;
                        tsum += e;
                    }
            } else {
                // The shift is the running max times |scale| log2(e), rounded once; alpha
                // compares two such rounded shifts, so an unchanged max gives exactly 1.
                const float c2 = p.scale_log2;
                const float shift = (m_new == kNegInf) ? 0.f : m_new * c2;
                alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run * c2 - shift);
                if (any_mask) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float e = keep[kb][r] ? fast_exp2(fmaf(s[kb][r], c2, -shift)) : 0.f;
                            s[kb][r] = e;
                            tsum += e;
                        }
                } else {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float e = fast_exp2(fmaf(s[kb][r], c2, -shift));
                            s[kb][r] = e;
                            tsum += e;
                        }
                }
            }
            m_run = m_new;
            l_run = fmaf(l_run, alpha, tsum);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    uint4 pb;
                    pb.x = Tr::pack2(s[kb][c * 8 + 0], s[kb][c * 8 + 1]);
                    pb.y = Tr::pack2(s[kb][c * 8 + 2], s[kb][c * 8 + 3]);
                    pb.z = Tr::pack2(s[kb][c * 8 + 4], s[kb][c * 8 + 5]);
                    pb.w = Tr::pack2(s[kb][c * 8 + 6], s[kb][c * 8 + 7]);
                    const int lchunk = kb * 4 + c * 2 + hh;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const int d = db * 32 + lq;
                        const uint4 a = *(const uint4*)(Vt + d * VS + ((lchunk ^ ((d >> 3) & 7)) * 8));
                        acc[db] = Tr::mfma32(as_vec8<Tr>(a), as_vec8<Tr>(pb), acc[db]);
                    }
                }
        }
        if (t + 1 < ntiles) store_tile((t + 1) & 1);
        __syncthreads();
    }

    // Epilogue: O = O^T / l per lane (this lane's query), rounded to nearest-even.
    const float l_tot = l_run + xor_lane(l_run, 32);
    if (my_row < Lb) {
        const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
        uint16_t* op = (uint16_t*)p.o + oo + (int64_t)my_row * p.o_sr;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + g * 8 + hh * 4;
                uint2 st;
                st.x = Tr::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv);
                st.y = Tr::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
                *(uint2*)(op + d) = st;
            }
        if (hh == 0) {
            float lse;
            if (l_tot == 0.f)
                lse = kNegInf;
            else if (MASK == MASK_FLOAT)
                lse = fmaf(fast_log2(l_tot), kLn2, m_run);
            else
                lse = (m_run * p.scale_log2 + fast_log2(l_tot)) * kLn2;
            p.lse[lo + my_row] = lse;
        }
    }
}

template <typename Tr, int D, bool CAUSAL, int MASK, bool VARLEN>
hipError_t launch_prefill_one(const AttnParams& p, hipStream_t stream) {
    const long long grid = (long long)p.n_qtiles * p.Hq * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_mfma_kernel<Tr, D, CAUSAL, MASK, VARLEN>), dim3((unsigned)grid),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename Tr, int D>
hipError_t launch_prefill_d(const AttnParams& p, bool causal, int mask, bool varlen,
                            hipStream_t s) {
    if (varlen) {
        if (mask != MASK_NONE) return hipErrorInvalidValue;
        return causal ? launch_prefill_one<Tr, D, true, MASK_NONE, true>(p, s)
                      : launch_prefill_one<Tr, D, false, MASK_NONE, true>(p, s);
    }
    switch (mask) {
        case MASK_NONE:
            return causal ? launch_prefill_one<Tr, D, true, MASK_NONE, false>(p, s)
                          : launch_prefill_one<Tr, D, false, MASK_NONE, false>(p, s);
        case MASK_FLOAT:
            return causal ? launch_prefill_one<Tr, D, true, MASK_FLOAT, false>(p, s)
                          : launch_prefill_one<Tr, D, false, MASK_FLOAT, false>(p, s);
        case MASK_BOOL:
            return causal ? launch_prefill_one<Tr, D, true, MASK_BOOL, false>(p, s)
                          : launch_prefill_one<Tr, D, false, MASK_BOOL, false>(p, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tr>
hipError_t launch_prefill_t(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                            hipStream_t s) {
    switch (D) {
        case 64: return launch_prefill_d<Tr, 64>(p, causal, mask, varlen, s);
        case 96: return launch_prefill_d<Tr, 96>(p, causal, mask, varlen, s);
        case 128: return launch_prefill_d<Tr, 128>(p, causal, mask, varlen, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sdpa

// Single-pass attention forward for fp32 inputs, on the vector ALUs.
//
// Same blocked online-softmax method as the matrix-core kernel (khchao.com NN
// Lab, "FlashAttention Tiling & Online Softmax Algorithm"), kept in fp32
// throughout: no input is rounded to a narrower format (no xf32/tf32).
//
// Layout: a workgroup of 256 lanes owns 64 query rows; four consecutive lanes
// share one row and each holds a quarter of its head dim, in 4-float runs
// interleaved with period 16.  A score is therefore 16 partial dot products
// (4 per lane) combined in a fixed tree, which keeps the rounding error of
// the E-long dot product well below that of one sequential FMA chain (the
// four lanes of a row combine theirs with quad DPP moves).  Keys and values
// stream through LDS 32 rows at a time, the next block's loads in flight in
// registers while a block is computed.  The running max is kept in logit
// units and subtracted before multiplying by log2(e).
//
// Padded instances (PADE): head dims E and Ev that are multiples of 8 up to 128
// (E = 0 included) run at a width D of 64 or 128: columns of Q and K from E on,
// and of V from Ev on, are never read and stand as 0 (the dot products only gain
// exact zeros), and output columns from Ev on are never written.
#include "attn_common.h"
#include "device_utils.h"

namespace sdpa {

template <int D, bool CAUSAL, int MASK, bool VARLEN, bool PADE = false>
__global__ __launch_bounds__(256) void prefill_f32_kernel(AttnParams p) {
    constexpr int BM = kF32BlockM;
    constexpr int BN = 32;
    constexpr int RS = D + 4;          // LDS row stride (floats)
    constexpr int NI = D / 16;         // float4 runs per lane
    constexpr int NCH = BN * D / 4;    // float4 chunks per tile
    __shared__ __attribute__((aligned(16))) float Ks[BN * RS];
    __shared__ __attribute__((aligned(16))) float Vs[BN * RS];

    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int rloc = tid >> 2;

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
        Sb = (int)min(d - c, (int64_t)p.S);  // at most max_seqlen_k, as the backward
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
    const int row = q0 + rloc;
    const bool valid = row < Lb;
    const int kend = CAUSAL ? min(Sb, min(q0 + BM, Lb)) : Sb;

    float4 qv[NI], ov[NI];
    const float* qp = (const float*)p.q + qo + (int64_t)min(row, Lb - 1) * p.q_sr;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const bool qin = valid && (!PADE || i * 16 + part * 4 < p.e);
        qv[i] = qin ? *(const float4*)(qp + i * 16 + part * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        ov[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float* mrow_f = (const float*)p.mask + mo + (int64_t)min(row, Lb - 1) * p.m_sr;
    const uint8_t* mrow_b = (const uint8_t*)p.mask + mo + (int64_t)min(row, Lb - 1) * p.m_sr;
    const float* kp = (const float*)p.k + ko;
    const float* vp = (const float*)p.v + vo;

    float m_run = kNegInf, l_run = 0.f;
    // the next block's keys and values travel in registers while this block
    // is computed (NCH / 256 chunks of each per lane)
    constexpr int NCT = (NCH + 255) / 256;
    float4 kb[NCT], vb[NCT];
    auto load_block = [&](int key0) {
#pragma unroll
        for (int i = 0; i < NCT; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (D / 4), col = (c % (D / 4)) * 4;
            const bool in = c < NCH && key0 + r < Sb;
            const bool kin = in && (!PADE || col < p.e);
            const bool vin = in && (!PADE || col < p.dv);
            kb[i] = kin ? *(const float4*)(kp + (int64_t)(key0 + r) * p.k_sr + col) : make_float4(0.f, 0.f, 0.f, 0.f);
            vb[i] = vin ? *(const float4*)(vp + (int64_t)(key0 + r) * p.v_sr + col) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    if (kend > 0) load_block(0);
    for (int key0 = 0; key0 < kend; key0 += BN) {
#pragma unroll
        for (int i = 0; i < NCT; ++i) {
            const int c = tid + 256 * i;
            if (c < NCH) {
                const int r = c / (D / 4), col = (c % (D / 4)) * 4;
                *(float4*)(Ks + r * RS + col) = kb[i];
                *(float4*)(Vs + r * RS + col) = vb[i];
            }
        }
        __syncthreads();
        if (key0 + BN < kend) load_block(key0 + BN);
        float lg[BN];
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float4 kv = *(const float4*)(Ks + j * RS + i * 16 + part * 4);
                a0 = fmaf(qv[i].x, kv.x, a0);
                a1 = fmaf(qv[i].y, kv.y, a1);
                a2 = fmaf(qv[i].z, kv.z, a2);
                a3 = fmaf(qv[i].w, kv.w, a3);
            }
            // the four lanes of a row exchange partial sums within their quad
            // (DPP quad permutations [1,0,3,2] and [2,3,0,1]); every lane ends
            // with the same (p0 + p1) + (p2 + p3)
            float sc = (a0 + a1) + (a2 + a3);
            sc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sc), 0xB1, 0xF, 0xF, false));
            sc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sc), 0x4E, 0xF, 0xF, false));
            const int key = key0 + j;
            float x;
            if (MASK == MASK_FLOAT)
                x = fmaf(sc, p.scale, key < Sb ? mrow_f[key] : 0.f);
            else
                x = sc * p.scale;
            bool keep = key < Sb;
            if (MASK == MASK_BOOL) keep = keep && mrow_b[key < Sb ? key : 0] != 0;
            if (CAUSAL) keep = keep && key <= row;
            lg[j] = keep ? x : kNegInf;
        }
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < BN; ++j) mx = fmaxf(mx, lg[j]);
        const float m_new = fmaxf(m_run, mx);
        const float shift = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = (m_run == kNegInf) ? 0.f : exp2f((m_run - m_new) * kLog2e);
        m_run = m_new;
        float tsum = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            ov[i].x *= alpha; ov[i].y *= alpha; ov[i].z *= alpha; ov[i].w *= alpha;
        }
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            const float e = exp2f((lg[j] - shift) * kLog2e);
            tsum += e;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float4 vv = *(const float4*)(Vs + j * RS + i * 16 + part * 4);
                ov[i].x = fmaf(e, vv.x, ov[i].x);
                ov[i].y = fmaf(e, vv.y, ov[i].y);
                ov[i].z = fmaf(e, vv.z, ov[i].z);
                ov[i].w = fmaf(e, vv.w, ov[i].w);
            }
        }
        l_run = fmaf(l_run, alpha, tsum);
        __syncthreads();
    }
    if (valid) {
        float* op = (float*)p.o + oo + (int64_t)row * p.o_sr;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float4 r;
            if (l_run == 0.f) {
                r = make_float4(ov[i].x * 0.f, ov[i].y * 0.f, ov[i].z * 0.f, ov[i].w * 0.f);
            } else {
                r = make_float4(ov[i].x / l_run, ov[i].y / l_run, ov[i].z / l_run, ov[i].w / l_run);
            }
            if (!PADE || i * 16 + part * 4 < p.dv) *(float4*)(op + i * 16 + part * 4) = r;
        }
        if (part == 0) p.lse[lo + row] = (l_run == 0.f) ? kNegInf : m_run + logf(l_run);
    }
}

template <int D, bool CAUSAL, int MASK, bool VARLEN, bool PADE>
static hipError_t launch_f32_one(const AttnParams& p, hipStream_t stream) {
    const long long grid = (long long)p.n_qtiles * p.Hq * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, MASK, VARLEN, PADE>), dim3((unsigned)grid), dim3(256),
                       0, stream, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool PADE>
static hipError_t launch_f32_c(const AttnParams& p, int mask, bool varlen, hipStream_t s) {
    if (varlen)
        return mask == MASK_NONE ? launch_f32_one<D, CAUSAL, MASK_NONE, true, PADE>(p, s) : hipErrorInvalidValue;
    switch (mask) {
        case MASK_NONE: return launch_f32_one<D, CAUSAL, MASK_NONE, false, PADE>(p, s);
        case MASK_FLOAT: return launch_f32_one<D, CAUSAL, MASK_FLOAT, false, PADE>(p, s);
        case MASK_BOOL: return launch_f32_one<D, CAUSAL, MASK_BOOL, false, PADE>(p, s);
    }
    return hipErrorInvalidValue;
}

template <int D, bool PADE>
static hipError_t launch_f32_d(const AttnParams& p, bool causal, int mask, bool varlen, hipStream_t s) {
    return causal ? launch_f32_c<D, true, PADE>(p, mask, varlen, s) : launch_f32_c<D, false, PADE>(p, mask, varlen, s);
}

hipError_t launch_prefill_f32(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                              hipStream_t s) {
    (void)D;
    if (p.e == p.dv) {
        switch (p.e) {
            case 64: return launch_f32_d<64, false>(p, causal, mask, varlen, s);
            case 96: return launch_f32_d<96, false>(p, causal, mask, varlen, s);
            case 128: return launch_f32_d<128, false>(p, causal, mask, varlen, s);
        }
    }
    if (p.e < 0 || p.e > 128 || p.e % 8 != 0 || p.dv < 0 || p.dv > 128 || p.dv % 8 != 0)
        return hipErrorInvalidValue;
    return max(p.e, p.dv) <= 64 ? launch_f32_d<64, true>(p, causal, mask, varlen, s)
                                : launch_f32_d<128, true>(p, causal, mask, varlen, s);
}

}  // namespace sdpa

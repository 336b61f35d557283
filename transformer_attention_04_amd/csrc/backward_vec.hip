// Gradients of attention on the vector ALUs in fp32 arithmetic, for the calls
// the matrix-core backward (backward.hip) does not take: fp32 inputs, value
// rows of another width than query/key rows (Ev != E), and head dims other
// than 64/96/128 (E and Ev multiples of 8 up to 128, E = 0 and Ev = 0
// included).  The formulas are those of the exactref.ai
// "scaled_dot_product_attention.backward" section: with P the attention
// weights, recomputed as exp(logit - lse) from the forward's logsumexp,
//     dP = grad V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
//     grad_value = P^T grad,  grad_query = scale dS K,  grad_key = scale dS^T Q,
// each summed over the query heads of a key/value group.  D_i is formed as
// dO_i . O_i from the forward's output (the same number in exact arithmetic,
// since O_i = sum_j P_ij V_j), as the matrix-core backward does.
//
// Two kernels, one owner per gradient element (no atomics, deterministic):
//   bwdv_dq_kernel    a workgroup per 32 query rows of one (batch, head): D of
//                     its rows (written to the workspace), then for each block
//                     of 32 keys the scores, dP and dS in LDS, and dQ += dS K;
//   bwdv_dkdv_kernel  a workgroup per 32 keys of one (batch, key/value head):
//                     for every query head of the group and block of 32 query
//                     rows (from the causal diagonal on), P and dS in LDS,
//                     dV += P^T dO and dK += dS^T Q.
// Tiles sit in LDS as fp32 with rows padded to 129 floats; every thread owns
// (row, column) pairs t % 8 + 8 m of one row t / 8, so the dot products read
// one LDS row broadcast to 8 threads and 8 consecutive columns.
// A row with no kept key has lse -inf: it is read as 0, so every weight of the
// row is exp(-inf) = 0 and the row contributes nothing, as the page specifies.
#include "attn_common.h"
#include "device_utils.h"

namespace sdpa {

constexpr int kVT = 32;    // query rows / keys per tile
constexpr int kVD = 128;   // widest head dim
constexpr int kVS = kVD + 1;

template <int ELEM>
__device__ __forceinline__ float ldv(const void* base, int64_t i) {
    if constexpr (ELEM == ELEM_F32) return ((const float*)base)[i];
    else if constexpr (ELEM == ELEM_BF16) return BF16::to_f32(((const uint16_t*)base)[i]);
    else return F16::to_f32(((const uint16_t*)base)[i]);
}

template <int ELEM>
__device__ __forceinline__ void stv(void* base, int64_t i, float x) {
    if constexpr (ELEM == ELEM_F32) ((float*)base)[i] = x;
    else if constexpr (ELEM == ELEM_BF16) ((uint16_t*)base)[i] = BF16::from_f32(x);
    else ((uint16_t*)base)[i] = F16::from_f32(x);
}

// Segment b of a packed batch (offsets clamped to the totals, lengths to L and S),
// or the whole (batch, head) rows of a batched call.
struct VSeg {
    int64_t a, c;   // first query token / key token (packed), else 0
    int Lb, Sb;
};

__device__ __forceinline__ VSeg vseg(const BwdParams& p, int b) {
    VSeg s;
    if (p.cu_q) {
        const int64_t a0 = min(max((int64_t)p.cu_q[b], (int64_t)0), p.total_q);
        const int64_t e0 = min(max((int64_t)p.cu_q[b + 1], a0), p.total_q);
        const int64_t c0 = min(max((int64_t)p.cu_k[b], (int64_t)0), p.total_k);
        const int64_t d0 = min(max((int64_t)p.cu_k[b + 1], c0), p.total_k);
        s.a = a0;
        s.c = c0;
        s.Lb = (int)min(e0 - a0, (int64_t)p.L);
        s.Sb = (int)min(d0 - c0, (int64_t)p.S);
    } else {
        s.a = s.c = 0;
        s.Lb = p.L;
        s.Sb = p.S;
    }
    return s;
}

// Element offsets of row r of head h in batch b (packed: token a + r).
__device__ __forceinline__ int64_t voff(const BwdParams& p, int64_t sb, int64_t sh, int64_t sr, int b, int h,
                                        int64_t a, int r) {
    return p.cu_q ? (a + r) * sr + (int64_t)h * sh : (int64_t)b * sb + (int64_t)h * sh + (int64_t)r * sr;
}

// Index of (b, h, row) in lse and in the D workspace.
__device__ __forceinline__ int64_t vlse(const BwdParams& p, int b, int h, int64_t a, int r) {
    return p.cu_q ? (int64_t)h * p.lse_sh + a + r : (int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + r;
}
__device__ __forceinline__ int64_t vdsum(const BwdParams& p, int b, int h, int64_t a, int r) {
    return p.cu_q ? (int64_t)h * p.total_q + a + r : ((int64_t)b * p.Hq + h) * p.L + r;
}

// logit of query row i (segment-local) and key j, or -inf when the key is dropped
template <int MASK, bool CAUSAL>
__device__ __forceinline__ float vlogit(const BwdParams& p, float s, int b, int h, int i, int j, int Sb) {
    if (j >= Sb || (CAUSAL && j > i)) return kNegInf;
    if constexpr (MASK == MASK_FLOAT) {
        const float bias = ((const float*)p.mask)[(int64_t)b * p.m_sb + (int64_t)h * p.m_sh + (int64_t)i * p.m_sr + j];
        return fmaf(s, p.scale, bias);
    } else if constexpr (MASK == MASK_BOOL) {
        const uint8_t keep = ((const uint8_t*)p.mask)[(int64_t)b * p.m_sb + (int64_t)h * p.m_sh + (int64_t)i * p.m_sr + j];
        return keep ? s * p.scale : kNegInf;
    } else {
        return s * p.scale;
    }
}

template <int ELEM, bool CAUSAL, int MASK>
__global__ __launch_bounds__(256) void bwdv_dq_kernel(BwdParams p) {
    __shared__ float Qs[kVT * kVS], Os[kVT * kVS], Ks[kVT * kVS], Vs[kVT * kVS], Ss[kVT * (kVT + 1)];
    __shared__ float Dsh[kVT], Lsh[kVT];
    const int tid = threadIdx.x;
    const int nbh = p.Hq * p.B;
    const int qt = (int)(blockIdx.x / nbh);
    const int bh = (int)(blockIdx.x % nbh);
    const int h = bh % p.Hq, b = bh / p.Hq, kvh = h / p.group;
    const VSeg sg = vseg(p, b);
    const int q0 = qt * kVT;
    if (q0 >= sg.Lb) return;
    const int rows = min(kVT, sg.Lb - q0);
    const int E = p.e, Ev = p.ev;
    const int r = tid >> 3, cl = tid & 7;   // this thread's row and column phase

    // Q and dO rows of the tile, D_i = dO_i . O_i, lse
    for (int x = tid; x < kVT * kVD; x += 256) {
        const int rr = x / kVD, c = x % kVD;
        const bool ok = rr < rows;
        Qs[rr * kVS + c] = ok && c < E ? ldv<ELEM>(p.q, voff(p, p.q_sb, p.q_sh, p.q_sr, b, h, sg.a, q0 + rr) + c) : 0.f;
        Os[rr * kVS + c] = ok && c < Ev ? ldv<ELEM>(p.dout, voff(p, p.do_sb, p.do_sh, p.do_sr, b, h, sg.a, q0 + rr) + c)
                                        : 0.f;
    }
    __syncthreads();
    {
        float d = 0.f;
        if (r < rows)
            for (int c = cl; c < Ev; c += 8)
                d = fmaf(Os[r * kVS + c], ldv<ELEM>(p.o, voff(p, p.o_sb, p.o_sh, p.o_sr, b, h, sg.a, q0 + r) + c), d);
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        d += __shfl_xor(d, 4, 64);
        if (cl == 0) {
            Dsh[r] = d;
            float l = r < rows ? p.lse[vlse(p, b, h, sg.a, q0 + r)] : 0.f;
            Lsh[r] = (l == kNegInf) ? 0.f : l;
            if (r < rows) p.dsum[vdsum(p, b, h, sg.a, q0 + r)] = d;
        }
    }
    float acc[kVD / 8];
#pragma unroll
    for (int m = 0; m < kVD / 8; ++m) acc[m] = 0.f;

    const int kend = CAUSAL ? min(sg.Sb, q0 + rows) : sg.Sb;
    for (int k0 = 0; k0 < kend; k0 += kVT) {
        __syncthreads();  // previous tile's readers are done
        for (int x = tid; x < kVT * kVD; x += 256) {
            const int j = x / kVD, c = x % kVD;
            const bool ok = k0 + j < sg.Sb;
            const int64_t kr = p.cu_q ? (sg.c + k0 + j) * p.k_sr + (int64_t)kvh * p.k_sh
                                      : (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + (int64_t)(k0 + j) * p.k_sr;
            const int64_t vr = p.cu_q ? (sg.c + k0 + j) * p.v_sr + (int64_t)kvh * p.v_sh
                                      : (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + (int64_t)(k0 + j) * p.v_sr;
            Ks[j * kVS + c] = ok && c < E ? ldv<ELEM>(p.k, kr + c) : 0.f;
            Vs[j * kVS + c] = ok && c < Ev ? ldv<ELEM>(p.v, vr + c) : 0.f;
        }
        __syncthreads();
        // scores, dP and dS for (row r, keys cl + 8m)
#pragma unroll
        for (int m = 0; m < kVT / 8; ++m) {
            const int j = cl + 8 * m;
            float s = 0.f, dp = 0.f;
            for (int c = 0; c < E; ++c) s = fmaf(Qs[r * kVS + c], Ks[j * kVS + c], s);
            for (int c = 0; c < Ev; ++c) dp = fmaf(Os[r * kVS + c], Vs[j * kVS + c], dp);
            const float lg = (r < rows) ? vlogit<MASK, CAUSAL>(p, s, b, h, q0 + r, k0 + j, sg.Sb) : kNegInf;
            const float pr = expf(lg - Lsh[r]);
            Ss[r * (kVT + 1) + j] = pr * (dp - Dsh[r]);
        }
        __syncthreads();
        // dQ += dS K for (row r, columns cl + 8m)
        for (int j = 0; j < kVT; ++j) {
            const float ds = Ss[r * (kVT + 1) + j];
#pragma unroll
            for (int m = 0; m < kVD / 8; ++m) acc[m] = fmaf(ds, Ks[j * kVS + cl + 8 * m], acc[m]);
        }
    }
    if (r < rows) {
        const int64_t o = voff(p, p.dq_sb, p.dq_sh, p.dq_sr, b, h, sg.a, q0 + r);
#pragma unroll
        for (int m = 0; m < kVD / 8; ++m) {
            const int c = cl + 8 * m;
            if (c < E) stv<ELEM>(p.dq, o + c, p.scale * acc[m]);
        }
    }
}

template <int ELEM, bool CAUSAL, int MASK>
__global__ __launch_bounds__(256) void bwdv_dkdv_kernel(BwdParams p) {
    __shared__ float Ks[kVT * kVS], Vs[kVT * kVS], Qs[kVT * kVS], Os[kVT * kVS];
    __shared__ float Ps[kVT * (kVT + 1)], Ss[kVT * (kVT + 1)], Dsh[kVT], Lsh[kVT];
    const int tid = threadIdx.x;
    const int nbh = p.Hkv * p.B;
    const int kt = (int)(blockIdx.x / nbh);
    const int bh = (int)(blockIdx.x % nbh);
    const int kvh = bh % p.Hkv, b = bh / p.Hkv;
    const VSeg sg = vseg(p, b);
    const int k0 = kt * kVT;
    if (k0 >= sg.Sb) return;
    const int keys = min(kVT, sg.Sb - k0);
    const int E = p.e, Ev = p.ev;
    const int r = tid >> 3, cl = tid & 7;   // r: a key of the tile (accumulators) or a query row (scores)

    for (int x = tid; x < kVT * kVD; x += 256) {
        const int j = x / kVD, c = x % kVD;
        const bool ok = j < keys;
        const int64_t kr = p.cu_q ? (sg.c + k0 + j) * p.k_sr + (int64_t)kvh * p.k_sh
                                  : (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + (int64_t)(k0 + j) * p.k_sr;
        const int64_t vr = p.cu_q ? (sg.c + k0 + j) * p.v_sr + (int64_t)kvh * p.v_sh
                                  : (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + (int64_t)(k0 + j) * p.v_sr;
        Ks[j * kVS + c] = ok && c < E ? ldv<ELEM>(p.k, kr + c) : 0.f;
        Vs[j * kVS + c] = ok && c < Ev ? ldv<ELEM>(p.v, vr + c) : 0.f;
    }
    float dk[kVD / 8], dv[kVD / 8];
#pragma unroll
    for (int m = 0; m < kVD / 8; ++m) dk[m] = dv[m] = 0.f;

    const int qstart = CAUSAL ? (k0 / kVT) * kVT : 0;
    for (int g = 0; g < p.group; ++g) {
        const int h = kvh * p.group + g;
        for (int q0 = qstart; q0 < sg.Lb; q0 += kVT) {
            const int rows = min(kVT, sg.Lb - q0);
            __syncthreads();  // previous block's readers are done
            for (int x = tid; x < kVT * kVD; x += 256) {
                const int rr = x / kVD, c = x % kVD;
                const bool ok = rr < rows;
                Qs[rr * kVS + c] = ok && c < E ? ldv<ELEM>(p.q, voff(p, p.q_sb, p.q_sh, p.q_sr, b, h, sg.a, q0 + rr) + c)
                                               : 0.f;
                Os[rr * kVS + c] = ok && c < Ev
                                       ? ldv<ELEM>(p.dout, voff(p, p.do_sb, p.do_sh, p.do_sr, b, h, sg.a, q0 + rr) + c)
                                       : 0.f;
            }
            if (tid < kVT) {
                const bool ok = tid < rows;
                Dsh[tid] = ok ? p.dsum[vdsum(p, b, h, sg.a, q0 + tid)] : 0.f;
                const float l = ok ? p.lse[vlse(p, b, h, sg.a, q0 + tid)] : 0.f;
                Lsh[tid] = (l == kNegInf) ? 0.f : l;
            }
            __syncthreads();
            // P and dS for (query row r, keys cl + 8m)
#pragma unroll
            for (int m = 0; m < kVT / 8; ++m) {
                const int j = cl + 8 * m;
                float s = 0.f, dp = 0.f;
                for (int c = 0; c < E; ++c) s = fmaf(Qs[r * kVS + c], Ks[j * kVS + c], s);
                for (int c = 0; c < Ev; ++c) dp = fmaf(Os[r * kVS + c], Vs[j * kVS + c], dp);
                const float lg = (r < rows) ? vlogit<MASK, CAUSAL>(p, s, b, h, q0 + r, k0 + j, sg.Sb) : kNegInf;
                const float pr = expf(lg - Lsh[r]);
                Ps[r * (kVT + 1) + j] = pr;
                Ss[r * (kVT + 1) + j] = pr * (dp - Dsh[r]);
            }
            __syncthreads();
            // dV += P^T dO, dK += dS^T Q for (key r, columns cl + 8m)
            for (int i = 0; i < kVT; ++i) {
                const float pr = Ps[i * (kVT + 1) + r], ds = Ss[i * (kVT + 1) + r];
#pragma unroll
                for (int m = 0; m < kVD / 8; ++m) {
                    dv[m] = fmaf(pr, Os[i * kVS + cl + 8 * m], dv[m]);
                    dk[m] = fmaf(ds, Qs[i * kVS + cl + 8 * m], dk[m]);
                }
            }
        }
    }
    if (r < keys) {
        const int64_t ko = p.cu_q ? (sg.c + k0 + r) * p.dk_sr + (int64_t)kvh * p.dk_sh
                                  : (int64_t)b * p.dk_sb + (int64_t)kvh * p.dk_sh + (int64_t)(k0 + r) * p.dk_sr;
        const int64_t vo = p.cu_q ? (sg.c + k0 + r) * p.dv_sr + (int64_t)kvh * p.dv_sh
                                  : (int64_t)b * p.dv_sb + (int64_t)kvh * p.dv_sh + (int64_t)(k0 + r) * p.dv_sr;
#pragma unroll
        for (int m = 0; m < kVD / 8; ++m) {
            const int c = cl + 8 * m;
            if (c < E) stv<ELEM>(p.dk, ko + c, p.scale * dk[m]);
            if (c < Ev) stv<ELEM>(p.dv, vo + c, dv[m]);
        }
    }
}

template <int ELEM, bool CAUSAL, int MASK>
static hipError_t launch_bwdv_one(const BwdParams& p, hipStream_t s) {
    const int nq = (p.L + kVT - 1) / kVT, nk = (p.S + kVT - 1) / kVT;
    const long long gq = (long long)nq * p.Hq * p.B, gk = (long long)nk * p.Hkv * p.B;
    if (gq > 0) hipLaunchKernelGGL((bwdv_dq_kernel<ELEM, CAUSAL, MASK>), dim3((unsigned)gq), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (gk > 0) hipLaunchKernelGGL((bwdv_dkdv_kernel<ELEM, CAUSAL, MASK>), dim3((unsigned)gk), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int ELEM>
static hipError_t launch_bwdv_e(const BwdParams& p, bool causal, int mask, hipStream_t s) {
    switch (mask) {
        case MASK_NONE: return causal ? launch_bwdv_one<ELEM, true, MASK_NONE>(p, s)
                                      : launch_bwdv_one<ELEM, false, MASK_NONE>(p, s);
        case MASK_FLOAT: return causal ? launch_bwdv_one<ELEM, true, MASK_FLOAT>(p, s)
                                       : launch_bwdv_one<ELEM, false, MASK_FLOAT>(p, s);
        case MASK_BOOL: return causal ? launch_bwdv_one<ELEM, true, MASK_BOOL>(p, s)
                                      : launch_bwdv_one<ELEM, false, MASK_BOOL>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_backward_vec(const BwdParams& p, bool causal, int mask, hipStream_t s) {
    if (p.e < 0 || p.e > kVD || p.ev < 0 || p.ev > kVD) return hipErrorInvalidValue;
    if (p.cu_q && mask != MASK_NONE) return hipErrorInvalidValue;
    switch (p.elem) {
        case ELEM_F32: return launch_bwdv_e<ELEM_F32>(p, causal, mask, s);
        case ELEM_BF16: return launch_bwdv_e<ELEM_BF16>(p, causal, mask, s);
        case ELEM_F16: return launch_bwdv_e<ELEM_F16>(p, causal, mask, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sdpa

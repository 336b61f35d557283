// Split-KV decode: attention of a few query rows over a long key/value cache.
//
// With one (or a handful of) new query tokens per sequence the work is
// dominated by streaming K and V from HBM once (khchao.com NN Lab, "Arithmetic
// Intensity of Autoregressive Decoding"); with grouped-query heads the query
// heads that share a key/value head read it together ("Memory Scaling
// Comparison: MHA vs MQA vs GQA").  The keys are cut into splits so the launch
// fills the chip; each split produces a normalised partial output O_s and its
// logsumexp lse_s over its own keys, and a merge pass combines them exactly:
//     lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s
// which follows from the definition of logsumexp over a partition of the keys
// (exactref.ai "scaled_dot_product_attention", Full specification, second
// output).  A split whose keys are all absent has lse_s = -inf and weight 0.
//
// gfx950 design of the split kernel (one workgroup = one (batch, kv head,
// split), 4 wavefronts; each wavefront takes 32-key sub-tiles in turn):
//  * scores S^T = K Q^T with v_mfma_f32_16x16x32: A = 16 keys x 32 dims loaded
//    straight from HBM into registers, B = the (<= 16) query rows of the
//    group, resident in registers; each lane ends with 4 keys of one query.
//  * the online-softmax max is reduced over the 4 lanes of a query column with
//    two lane exchanges; the weights go to a small per-wavefront LDS table.
//  * P V runs on the vector ALUs in fp32: each lane owns one 16-byte column
//    chunk of 8 keys' V rows (fully coalesced 256-byte row reads), reads the
//    weights of its keys from LDS and accumulates rows x 8 outputs.
//  * at the end the 4 lane groups and the 4 wavefronts are combined through
//    LDS into one normalised partial per query row.
//  * value rows may be narrower or wider than query/key rows (Ev != E: the
//    V chunks, partial outputs and merge use Ev); a paged cache variant reads
//    K/V through a block table (pages of >= 16 keys, one buffer resource per
//    16-key half, the split's page indices held in the lanes of a wavefront).
#include "attn_common.h"
#include "device_utils.h"

namespace sdpa {

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename Tr, int D, int DV, int NR, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    constexpr int NKK = D / 32;   // k-steps of the 16x16x32 score product
    constexpr int NDC = DV / 8;   // 16-byte chunks of a V row
    static_assert(NDC <= 16, "one chunk per lane of a 16-lane group");
    static_assert(NR % 4 == 0 && NR <= 16, "rows padded to 4, 8 or 16");

    __shared__ __attribute__((aligned(16))) float Pl[4][32 * NR];
    __shared__ __attribute__((aligned(16))) float Al[4][NR];
    __shared__ __attribute__((aligned(16))) float Ow[4][NR * DV];
    __shared__ float Mw[4][NR];
    __shared__ float Lw[4][NR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;     // query column (scores) / V column chunk (P V)
    const int grp = lane >> 4;   // which 4-key group (scores) / key row (P V)
    const int split = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    int seq = p.S;  // keys of this sequence
    if (PAGED) seq = max(0, min(p.S, min(p.seq_lens[b], p.max_blocks << p.page_shift)));
    const int ks = split * p.keys_per_split;
    const int ke = min(seq, ks + p.keys_per_split);
    const float c2 = p.scale_log2;
    // Last key + 1 kept for this lane's query column: all of the split, or
    // (paged, causal) up to the row's own position seq - L + i.
    int lim = ke;
    if (PAGED && p.causal && n < p.rows) lim = min(ke, seq - p.L + n / p.group + 1);
    // Paged: lane l holds the page of the split's l-th block (the host keeps a
    // split within 64 blocks).
    int pgv = 0;
    if (PAGED && ke > ks) {
        const int pb0 = ks >> p.page_shift;
        const int npg = ((ke - 1) >> p.page_shift) - pb0 + 1;
        if (lane < npg) pgv = p.block_table[(int64_t)b * p.bt_stride + pb0 + lane];
    }

    uint4 qreg[NKK];
    {
        const bool nvalid = n < p.rows;
        const int i = n / p.group, g = n % p.group;
        const int hq = kvh * p.group + g;
        const uint16_t* qp = (const uint16_t*)p.q + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh +
                             (int64_t)i * p.q_sr;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qreg[kk] = nvalid ? *(const uint4*)(qp + kk * 32 + grp * 8) : zero4();
        // negated after all loads are issued (a select per load would wait for each in turn)
        if (p.neg) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) qreg[kk] = negate8(qreg[kk]);
        }
    }
    const uint16_t* kp = (const uint16_t*)p.k + (int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh;
    const uint16_t* vp = (const uint16_t*)p.v + (int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh;

    float acc[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    // This split's keys through buffer resources: keys past the split read as 0.
    const int nk = max(ke - ks, 0);
    const int k_rs = (int)(p.k_sr * 2), v_rs = (int)(p.v_sr * 2);
    const auto kr = make_rsrc(kp + (int64_t)ks * p.k_sr, (nk - 1) * k_rs + D * 2);
    const auto vr = make_rsrc(vp + (int64_t)ks * p.v_sr, (nk - 1) * v_rs + DV * 2);
    // bad (paged): bit h set when keys key0 + 16h .. +15 include kept keys whose
    // table entry lies outside the page pool; nothing is read for them.
    auto load = [&](int key0, uint4 (&ka)[2][NKK], uint4 (&va)[8], int& bad) {
        bad = 0;
        if constexpr (!PAGED) {
            const int lk = key0 - ks;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
                    ka[kb][kk] = buf_load16(kr, (lk + kb * 16 + n) * k_rs + (kk * 32 + grp * 8) * 2);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                va[i] = buf_load16(vr, n < NDC ? (lk + grp + 4 * i) * v_rs + n * 16 : 0x7ffffff0);
        } else {
            // each half of the 32-key sub-tile lies in one page (pages hold >= 16 keys)
            __amdgpu_buffer_rsrc_t krh[2], vrh[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k16 = key0 + 16 * h;
                int nv = min(16, ke - k16);
                const int slot = min(63, max(0, (k16 >> p.page_shift) - (ks >> p.page_shift)));
                const int pg = __builtin_amdgcn_readlane(pgv, slot);
                const bool okp = (unsigned)pg < (unsigned)p.n_pages;
                if (!okp && nv > 0) bad |= 1 << h;
                if (!okp) nv = 0;
                const int64_t row0 = (int64_t)(okp ? pg : 0) * p.k_sb + (int64_t)kvh * p.k_sh +
                                     (int64_t)(k16 & ((1 << p.page_shift) - 1)) * p.k_sr;
                const int64_t vrow0 = (int64_t)(okp ? pg : 0) * p.v_sb + (int64_t)kvh * p.v_sh +
                                      (int64_t)(k16 & ((1 << p.page_shift) - 1)) * p.v_sr;
                krh[h] = make_rsrc((const uint16_t*)p.k + row0, (nv - 1) * k_rs + D * 2);
                vrh[h] = make_rsrc((const uint16_t*)p.v + vrow0, (nv - 1) * v_rs + DV * 2);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
                    ka[kb][kk] = buf_load16(krh[kb], n * k_rs + (kk * 32 + grp * 8) * 2);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                va[i] = buf_load16(vrh[i >> 2], n < NDC ? (grp + 4 * (i & 3)) * v_rs + n * 16 : 0x7ffffff0);
        }
    };
    // One 32-key sub-tile: scores, online softmax, P V.
    auto compute = [&](int key0, const uint4 (&ka)[2][NKK], const uint4 (&va)[8], int bad) {
        f32x4_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x4_t{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                s[kb] = Tr::mfma16(as_vec8<Tr>(ka[kb][kk]), as_vec8<Tr>(qreg[kk]), s[kb]);
        }
        // s[kb][i]: score of key key0 + 16kb + 4grp + i for query column n
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kept = key0 + kb * 16 + grp * 4 + i < lim;
                if (!kept) s[kb][i] = kNegInf;
                if (PAGED && ((bad >> kb) & 1) && kept) s[kb][i] = __builtin_nanf("");
                mx = fmaxf(mx, s[kb][i]);
            }
        mx = fmaxf(mx, xor_lane(mx, 16));
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float shift = (m_new == kNegInf) ? 0.f : m_new * c2;
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run * c2 - shift);
        m_run = m_new;
        float tsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kl = kb * 16 + grp * 4 + i;
                const float e = (key0 + kl < lim) ? fast_exp2(fmaf(s[kb][i], c2, -shift)) : 0.f;
                tsum += e;
                if (n < NR) Pl[wave][kl * NR + n] = e;
            }
        l_run = fmaf(l_run, alpha, tsum);
        if (grp == 0 && n < NR) Al[wave][n] = alpha;
        wave_lds_sync();

        float al[NR];
#pragma unroll
        for (int r = 0; r < NR; r += 4) {
            const float4 a4 = *(const float4*)(&Al[wave][r]);
            al[r] = a4.x; al[r + 1] = a4.y; al[r + 2] = a4.z; al[r + 3] = a4.w;
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= al[r];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kl = grp + 4 * i;
            float pr[NR];
#pragma unroll
            for (int r = 0; r < NR; r += 4) {
                const float4 p4 = *(const float4*)(&Pl[wave][kl * NR + r]);
                pr[r] = p4.x; pr[r + 1] = p4.y; pr[r + 2] = p4.z; pr[r + 3] = p4.w;
            }
            const uint32_t* w = (const uint32_t*)&va[i];
            float vf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[2 * e] = Tr::to_f32((uint16_t)(w[e] & 0xffffu));
                vf[2 * e + 1] = Tr::to_f32((uint16_t)(w[e] >> 16));
            }
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pr[r], vf[e], acc[r][e]);
        }
        wave_lds_sync();
    };
    // Each wavefront takes every fourth 32-key sub-tile; the next one's K and V
    // are in flight while the current one is computed.
    uint4 kaA[2][NKK], vaA[8], kaB[2][NKK], vaB[8];
    int badA = 0, badB = 0;
    int key0 = ks + wave * 32;
    if (key0 < ke) load(key0, kaA, vaA, badA);
    for (; key0 < ke; key0 += 256) {
        if (key0 + 128 < ke) load(key0 + 128, kaB, vaB, badB);
        compute(key0, kaA, vaA, badA);
        if (key0 + 128 >= ke) break;
        if (key0 + 256 < ke) load(key0 + 256, kaA, vaA, badA);
        compute(key0 + 128, kaB, vaB, badB);
    }

    // Combine the 4 lane groups (same column chunk, different keys) ...
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[r][e];
            x += xor_lane(x, 16);
            x += xor_lane(x, 32);
            acc[r][e] = x;
        }
    l_run += xor_lane(l_run, 16);
    l_run += xor_lane(l_run, 32);
    if (grp == 0) {
        if (n < NDC) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) Ow[wave][r * DV + n * 8 + e] = acc[r][e];
        }
        if (n < NR) {
            Mw[wave][n] = m_run;
            Lw[wave][n] = l_run;
        }
    }
    __syncthreads();

    // ... then the 4 wavefronts, into one normalised partial per query row.
    for (int idx = tid; idx < p.rows * DV; idx += 256) {
        const int r = idx / DV, d = idx % DV;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, Mw[w][r]);
        const float shift = (M == kNegInf) ? 0.f : M * c2;
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float a = (Mw[w][r] == kNegInf) ? 0.f : fast_exp2(Mw[w][r] * c2 - shift);
            L = fmaf(a, Lw[w][r], L);
            o = fmaf(a, Ow[w][r * DV + d], o);
        }
        const int i = r / p.group, g = r % p.group;
        const int hq = kvh * p.group + g;
        const int64_t prow = (((int64_t)b * p.Hq + hq) * p.L + i) * p.n_splits + split;
        p.part_o[prow * DV + d] = (L == 0.f) ? 0.f : o / L;
        if (d == 0) p.part_lse[prow] = (L == 0.f) ? kNegInf : (shift + fast_log2(L)) * kLn2;
    }
}

template <typename Tr, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p) {
    const int row = blockIdx.x;  // (b, hq, i) flattened
    const int i = row % p.L;
    const int hq = (row / p.L) % p.Hq;
    const int b = row / (p.L * p.Hq);
    const float* pl = p.part_lse + (int64_t)row * p.n_splits;
    float M = kNegInf;
    for (int s = 0; s < p.n_splits; ++s) M = fmaxf(M, pl[s]);
    const float shift = (M == kNegInf) ? 0.f : M;
    float W = 0.f;
    for (int s = 0; s < p.n_splits; ++s) W += fast_exp2((pl[s] - shift) * kLog2e);
    uint16_t* op = (uint16_t*)p.o + (int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)i * p.o_sr;
    const float* po = p.part_o + (int64_t)row * p.n_splits * D;
    for (int d = threadIdx.x; d < D; d += 64) {
        float o = 0.f;
        for (int s = 0; s < p.n_splits; ++s)
            o = fmaf(fast_exp2((pl[s] - shift) * kLog2e), po[(int64_t)s * D + d], o);
        op[d] = Tr::from_f32(W == 0.f ? 0.f : o / W);
    }
    if (threadIdx.x == 0)
        p.lse[(int64_t)b * p.lse_sb + (int64_t)hq * p.lse_sh + i] =
            (W == 0.f) ? kNegInf : fmaf(fast_log2(W), kLn2, shift);
}

template <typename Tr, int D, int DV>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t s) {
    dim3 grid(p.n_splits, p.Hkv, p.B);
    if (p.block_table) {
        if (p.rows <= 4)
            hipLaunchKernelGGL((decode_split_kernel<Tr, D, DV, 4, true>), grid, dim3(256), 0, s, p);
        else if (p.rows <= 8)
            hipLaunchKernelGGL((decode_split_kernel<Tr, D, DV, 8, true>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((decode_split_kernel<Tr, D, DV, 16, true>), grid, dim3(256), 0, s, p);
        goto merge;
    }
    if (p.rows <= 4)
        hipLaunchKernelGGL((decode_split_kernel<Tr, D, DV, 4, false>), grid, dim3(256), 0, s, p);
    else if (p.rows <= 8)
        hipLaunchKernelGGL((decode_split_kernel<Tr, D, DV, 8, false>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<Tr, D, DV, 16, false>), grid, dim3(256), 0, s, p);
merge:
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long nrows = (long long)p.B * p.Hq * p.L;
    hipLaunchKernelGGL((decode_merge_kernel<Tr, DV>), dim3((unsigned)nrows), dim3(64), 0, s, p);
    return hipGetLastError();
}

template <typename Tr, int D>
static hipError_t launch_decode_dv(const DecodeParams& p, hipStream_t s) {
    switch (p.dv) {
        case 64: return launch_decode_d<Tr, D, 64>(p, s);
        case 96: return launch_decode_d<Tr, D, 96>(p, s);
        case 128: return launch_decode_d<Tr, D, 128>(p, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tr>
static hipError_t launch_decode_t(const DecodeParams& p, int D, hipStream_t s) {
    switch (D) {
        case 64: return launch_decode_dv<Tr, 64>(p, s);
        case 96: return launch_decode_dv<Tr, 96>(p, s);
        case 128: return launch_decode_dv<Tr, 128>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int elem, int D, hipStream_t s) {
    if ((long long)p.B * p.Hkv * p.n_splits == 0 || p.L == 0) return hipSuccess;
    if (elem == ELEM_BF16) return launch_decode_t<BF16>(p, D, s);
    if (elem == ELEM_F16) return launch_decode_t<F16>(p, D, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa

// Single-pass attention forward for bf16 / fp16 inputs on gfx950, scheduled as
// two wavefront groups in lock step ("ping-pong").
//
// Method: the blocked, online-softmax form of exact attention described on the
// khchao.com NN Lab page ("FlashAttention Tiling & Online Softmax Algorithm");
// the result is softmax(scale * Q K^T + mask) V with its logsumexp, as the
// exactref.ai "scaled_dot_product_attention" Full specification defines it.
//
// Why this schedule.  On gfx950 a single wavefront issues a plain vector
// instruction only every ~4-6 cycles and an exponential every ~9, so the
// softmax of a 64-key block (about 150 vector instructions for 32 query rows)
// occupies one wavefront about as long as its 32 matrix instructions keep the
// matrix core busy (32 cycles each at E = 128); the vector work that does not
// depend on the block's row max is therefore done between matrix instructions.  A workgroup is therefore 8 wavefronts (256 query
// rows, 32 per wavefront); waves w and w + 4 share a SIMD.  Waves 0-3 (group A)
// and 4-7 (group B) run the same two-slot program, group B one slot behind,
// with a workgroup barrier between slots:
//
//   slot X(t)  S^T = K Q^T of block t, then O^T += V^T P^T of block t - 1
//              (32 MFMAs, operands read from LDS two products ahead of use);
//              between the score products the weights of block t - 1 are
//              packed to P^T and summed into the row sum
//   slot Y(t)  row max and lazy shift of block t, its unnormalised weights
//              (32 exponentials), the O rescale when the shift moved;
//              direct-to-LDS loads of block t + 3
//
// so while one wavefront of a SIMD issues matrix instructions the other does
// its vector and memory work.  Every barrier is preceded by a wait for the
// wave's own LDS reads, so a buffer may be overwritten one slot after its last
// reader's barrier.
//
// Key and value blocks travel HBM -> LDS by direct-to-LDS buffer loads (no
// staging registers, no LDS write instructions) into a ring of 4 stages:
// group A loads K, group B loads V, three blocks ahead.  Each lane of a load
// chooses which global 16-byte chunk lands in its LDS slot, so the layouts are
// free permutations of chunks, picked to make every operand read free of bank
// conflicts (64 banks; 16-byte reads serviced 16 lanes at a time, 8-byte reads
// 32 at a time, as measured on gfx950):
//   K: rows in groups of 16; within a group, chunk-major ([chunk][row]), so
//      the 16 lanes reading one chunk of 16 rows touch 256 contiguous bytes.
//      Row r of the block lands at LDS row swap23(r) (bits 2 and 3 of the
//      index swapped) so the score registers are the P^T operand of the
//      second product in k-slot order.
//   V: keys in groups of 4; within a group, [chunk][key].  The V^T operand
//      is read with ds_read_b64_tr_b16: within 16 lanes, lane i receives
//      column i of a 4 x 16 block assembled from four lanes' 8-byte reads, so
//      each lane gets 4 consecutive keys of one head-dimension column.
// Scores are transposed (one query per lane), the running max is lazy, and
// buffer resources turn reads past the last key into zeros.
//
// Timing of block t's stage (A runs slot k in phase k + 1, B in phase k + 2,
// slots numbered X(0) = 0, Y(0) = 1, X(1) = 2, ...): loaded in Y(t - 3) (phases
// 2t - 4 for K by A, 2t - 3 for V by B); each wave waits for its loads at the
// end of its Y(t - 1) (phases 2t and 2t + 1); K is read in X(t) (phases 2t + 1,
// 2t + 2) and V in X(t + 1) (phases 2t + 3, 2t + 4); block t + 4 is loaded into
// the same stage in Y(t + 1) (phases 2t + 4 and 2t + 5): the V reads of block t
// by group B share phase 2t + 4 with the K loads by group A, which is why K
// and V sit in separate halves of a stage and the ring has four stages.
// The per-wave register state between slots: the scores s of block t
// (X(t) -> Y(t)), its weights e and rescale factor (Y(t) -> X(t + 1)), O^T.
#pragma once

#include "attn_common.h"
#include "device_utils.h"

#include <type_traits>

namespace sdpa {

constexpr int kPPBlockM = 256;  // query rows per ping-pong workgroup

// Swap bits 2 and 3 of a key index within its 32-key block.
__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Exponent margin (log2 units) by which a block max may exceed the current
// shift before the shift is raised.
constexpr float kLazyRescale = 8.0f;

// End of a slot: this wave's LDS accesses, and all but VM of its direct-to-LDS
// loads, have completed; then all 8 waves meet.  The empty asm statements with
// a memory clobber keep the compiler from moving memory accesses across, the
// scheduling barriers keep it from moving any instruction across.
template <int VM>
__device__ __forceinline__ void pp_barrier() {
    static_assert(VM >= 0 && VM < 16, "vmcnt immediate");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | VM);  // vmcnt(VM) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void pp_barrier_lds() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// One direct-to-LDS load: lane m's 16 bytes at byte offset voff of the buffer
// land at LDS byte address m0 + 16 m.  Written as asm so that the compiler does
// not track it; the waits for it are the explicit ones at slot barriers.  The
// load has no register result.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; no compiler code here uses it
__device__ __forceinline__ void pp_dma16(u32x4_t rsrc, int voff, uint32_t m0) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(m0)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer resource as four scalars (for the asm operand).
__device__ __forceinline__ u32x4_t pp_rsrc(const void* base, int bytes) {
    const uint64_t a = (uint64_t)base;
    u32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu;
    r.z = __builtin_amdgcn_readfirstlane((uint32_t)max(bytes, 0));
    r.w = kRawBufferWord3;
    return r;
}

template <typename Tr, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_pp_kernel(AttnParams p) {
    constexpr int BM = kPPBlockM;
    constexpr int BN = 64;
    constexpr int NC = D / 8;          // 16-byte chunks per row
    constexpr int KTILE = BN * D;      // one K or V block, 16-bit words
    constexpr int NSTAGE = 4;          // ring of K/V stages
    constexpr int STAGE = 2 * KTILE;   // K block then V block
    constexpr int NKK = D / 16;        // k-steps of the score product
    constexpr int NDB = D / 32;        // 32-row blocks of O^T
    constexpr int NDMA = NC / 4;       // direct-to-LDS loads per wave per block
    static_assert(D == 64 || D == 96 || D == 128, "head dim must be 64, 96 or 128");
    static_assert(2 * NKK == 4 * NDB, "one K operand read per P.V product");

    __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int grp = wave >> 2;     // 0: group A, 1: group B (one slot behind)
    const int wg = wave & 3;
    const int lq = lane & 31;
    const int hh = lane >> 5;

    const int nbh = p.Hq * p.B;
    const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / nbh);
    const int bh = (int)(blockIdx.x % nbh);
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int kvh = h / p.group;

    int Lb, Sb;
    int64_t qo, ko, vo, oo, lo;
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
    }
    const int q0 = qt * BM;
    if (q0 >= Lb) return;  // whole workgroup, before any barrier
    const int kend = CAUSAL ? min(Sb, min(q0 + BM, Lb)) : Sb;
    const int ntiles = (kend + BN - 1) / BN;
    const int qrows = min(BM, Lb - q0);
    const int wrow0 = wave * 32;
    const int lrow = wrow0 + lq;
    const int my_row = q0 + lrow;
    const bool wave_has_rows = wrow0 < qrows;
    // last key block this wave takes part in (causal: its last row's block)
    const int last_tile = !wave_has_rows ? -1
                          : CAUSAL ? min(ntiles - 1, (q0 + wrow0 + 31) / BN)
                                   : ntiles - 1;

    // Q^T operand, resident for the whole loop (negated when the scale is negative).
    uint4 qreg[NKK];
    {
        const int q_rs = (int)(p.q_sr * 2);
        const auto qrs = make_rsrc((const uint16_t*)p.q + qo + (int64_t)q0 * p.q_sr, (qrows - 1) * q_rs + D * 2);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const uint4 u = buf_load16(qrs, lrow * q_rs + (kk * 16 + hh * 8) * 2);
            qreg[kk] = p.neg ? negate8(u) : u;
        }
    }

    // Direct-to-LDS loads of a block: group A moves K, group B moves V, NDMA
    // loads of 64 chunks per wave.  g_off[i] is the global byte offset (within
    // the block) of the chunk this lane places for load i.
    const int k_rs = (int)(p.k_sr * 2);
    const int v_rs = (int)(p.v_sr * 2);
    int g_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int P = (wg * NDMA + i) * 64 + lane;  // LDS chunk position in the block
        if (grp == 0) {
            const int r = (P / (16 * NC)) * 16 + P % 16, c = (P % (16 * NC)) / 16;
            const int row = (r & ~31) | swap_bits23(r & 31);
            g_off[i] = row * k_rs + c * 16;
        } else {
            const int k = (P / (4 * NC)) * 4 + P % 4, c = (P % (4 * NC)) / 4;
            g_off[i] = k * v_rs + c * 16;
        }
    }
    const int g_rs = grp == 0 ? k_rs : v_rs;
    const int64_t g_sr = grp == 0 ? p.k_sr : p.v_sr;
    const uint16_t* g_base = (const uint16_t*)(grp == 0 ? p.k : p.v) + (grp == 0 ? ko : vo);
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
    auto load_block = [&](int t) {
        const int key0 = t * BN;
        const int rows = min(BN, Sb - key0);
        const u32x4_t rs = pp_rsrc(g_base + (int64_t)key0 * g_sr, (rows - 1) * g_rs + D * 2);
        const uint32_t dst = smem_addr + (uint32_t)(((t % NSTAGE) * STAGE + grp * KTILE) * 2 + wg * NDMA * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) pp_dma16(rs, g_off[i], dst + i * 1024);
    };
    // End of slot Y(t): the loads of block t + 1 must have landed; those of
    // blocks t + 2 and t + 3 (issued in Y(t - 1) and Y(t) when they exist;
    // blocks 0-2 come from the prologue) may still be in flight.
    auto barrier_y = [&](int t) {
        const int newer = (t + 2 >= 3 && t + 2 < ntiles ? 1 : 0) + (t + 3 < ntiles ? 1 : 0);
        if (newer == 2)
            pp_barrier<2 * NDMA>();
        else if (newer == 1)
            pp_barrier<NDMA>();
        else
            pp_barrier<0>();
    };

    // K operand: LDS row kb*32 + lq, chunk kk*2 + hh -> position
    // (row/16)*16*NC + chunk*16 + row%16.
    const int k_lane = ((lq >> 4) * 16 * NC + hh * 16 + (lq & 15)) * 16;  // bytes
    // V^T operand of chunk ch (keys ch*16 + 8hh + 0..7), rows db*32 + 0..31:
    // two transposing reads of 4 keys each.  Lane i of a 16-lane group reads
    // key k0 + i/4, columns d0 + 4(i%4) .. +3, where d0 = db*32 + 16*(lane/16 & 1).
    const int vi = lane & 15;
    const int v_lane = ((hh * 2) * 4 * NC + (2 * ((lane >> 4) & 1) + (vi & 3) / 2) * 4 + vi / 4) * 16 + (vi & 1) * 8;

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    float sh_run = kNegInf;  // running shift, log2 units (-inf until a kept key)
    float l_run = 0.f;       // this lane's share of the row sum relative to it
    const float cfac = p.scale_log2;
    f32x16_t s[2];           // scores of block t, from X(t) to Y(t)
    f32x16_t e[2];           // unnormalised weights of block t, from Y(t) to X(t + 1)
    float alpha_e = 1.f;     // the rescale factor that came with e

    typedef short s16x4 __attribute__((ext_vector_type(4)));
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // V^T operand j = (chunk ch, 32 rows db) of block t: keys ch*16 + 8hh + 0..7,
    // two transposing reads of 4 keys each.
    auto read_v = [&](int t, int j) {
        const int ch = j / NDB, db = j % NDB;
        const char* Vb = (const char*)(smem + (t % NSTAGE) * STAGE + KTILE) + v_lane;
        const char* a0 = Vb + ((ch * 4 + 0) * 4 * NC + db * 16) * 16;
        const char* a1 = Vb + ((ch * 4 + 1) * 4 * NC + db * 16) * 16;
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(uint32_t)(uintptr_t)a0);
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(uint32_t)(uintptr_t)a1);
        uint4 u;
        u.x = __builtin_bit_cast(uint2, lo4).x;
        u.y = __builtin_bit_cast(uint2, lo4).y;
        u.z = __builtin_bit_cast(uint2, hi4).x;
        u.w = __builtin_bit_cast(uint2, hi4).y;
        return u;
    };
    auto read_k = [&](int t, int i) {  // K operand i = (kk = i/2, kb = i%2) of block t
        const char* Kb = (const char*)(smem + (t % NSTAGE) * STAGE) + k_lane;
        return *(const uint4*)(Kb + ((i & 1) * 2 * 16 * NC + (i >> 1) * 2 * 16) * 16);
    };

    // Slot X(t): S^T = K Q^T of block t, with the weights of block t - 1 packed
    // to P^T and summed in the gaps; then O^T += V^T P^T of block t - 1 (when PV
    // is set).  Operands stream from LDS two products ahead of their use, in
    // fenced order, so few are live at once.
    constexpr int NOP = 2 * NKK;  // products per half (16 at E = 128)
    static_assert(NOP == 4 * NDB, "one K operand read per P.V product");
    auto slot_x = [&](int t, auto pv_tag) {
        constexpr bool PV = decltype(pv_tag)::value;
        uint4 kop[NOP];
        uint4 pb[4];
        float p8[8];
        kop[0] = read_k(t, 0);
        kop[1] = read_k(t, 1);
        s[0] = f32x16_t{};
        s[1] = f32x16_t{};
        fence();
#pragma unroll
        for (int j = 0; j < NOP; ++j) {
            if (j + 2 < NOP) kop[j + 2] = read_k(t, j + 2);
            fence();
            s[j & 1] = Tr::mfma32(as_vec8<Tr>(kop[j]), as_vec8<Tr>(qreg[j >> 1]), s[j & 1]);
            if (PV) {
                // vector work of block t - 1 between the products: 13 items
                // (4 packs, 8 partial sums, the row-sum update) spread evenly
                // over the NOP products
#pragma unroll
                for (int w = (j * 13) / NOP; w < ((j + 1) * 13) / NOP; ++w) {
                    if (w < 4) {
                        const int kb = w >> 1, c = w & 1;
                        uint4 u;
                        u.x = Tr::pack2(e[kb][c * 8 + 0], e[kb][c * 8 + 1]);
                        u.y = Tr::pack2(e[kb][c * 8 + 2], e[kb][c * 8 + 3]);
                        u.z = Tr::pack2(e[kb][c * 8 + 4], e[kb][c * 8 + 5]);
                        u.w = Tr::pack2(e[kb][c * 8 + 6], e[kb][c * 8 + 7]);
                        pb[kb * 2 + c] = u;
                    } else if (w < 12) {
                        const int i = w - 4;
                        p8[i] = (e[i >> 2][(i & 3) * 4 + 0] + e[i >> 2][(i & 3) * 4 + 1]) +
                                (e[i >> 2][(i & 3) * 4 + 2] + e[i >> 2][(i & 3) * 4 + 3]);
                    } else {
                        const float tsum = ((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]));
                        l_run = fmaf(l_run, alpha_e, tsum);
                    }
                }
            }
            fence();
        }
        if (PV) {
            uint4 vop[NOP];
            vop[0] = read_v(t - 1, 0);
            vop[1] = read_v(t - 1, 1);
            fence();
#pragma unroll
            for (int j = 0; j < NOP; ++j) {
                if (j + 2 < NOP) vop[j + 2] = read_v(t - 1, j + 2);
                fence();
                acc[j % NDB] = Tr::mfma32(as_vec8<Tr>(vop[j]), as_vec8<Tr>(pb[j / NDB]), acc[j % NDB]);
                fence();
            }
        }
    };

    // Slot Y(t): row max and shift of block t, its unnormalised weights e;
    // the O rescale when the shift moved.  Exponentials are issued 16 at a time
    // on independent operands (fenced groups).
    auto slot_y = [&](int t) {
        const int key0 = t * BN;
        // s[kb][8c + j] is the score of key key0 + 32kb + 16c + 8hh + j for query my_row.
        const bool edge = (key0 + BN > Sb) || (CAUSAL && key0 + BN - 1 > q0 + wrow0);
        int lim = Sb - (key0 + hh * 8);
        if (CAUSAL) lim = min(lim, my_row + 1 - (key0 + hh * 8));
        float alpha = 1.f;
        auto softmax = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            if (MASKED) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int li = kb * 32 + (r >> 3) * 16 + (r & 7);
                        s[kb][r] = li < lim ? s[kb][r] : kNegInf;
                    }
            }
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
            const float mxs = mx * cfac;
            const bool raise = mxs > sh_run + kLazyRescale;
            const float sh_new = raise ? mxs : sh_run;
            alpha = raise ? fast_exp2(sh_run - sh_new) : 1.f;
            sh_run = sh_new;
            const float shift = (sh_new == kNegInf) ? 0.f : sh_new;
            fence();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) e[kb][r] = fmaf(s[kb][r], cfac, -shift);
                fence();
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float w = fast_exp2(e[kb][r]);
                    // masked keys by index (not by the score)
                    if (MASKED) w = (kb * 32 + (r >> 3) * 16 + (r & 7)) < lim ? w : 0.f;
                    e[kb][r] = w;
                }
                fence();
            }
        };
        if (edge)
            softmax(std::integral_constant<bool, true>{});
        else
            softmax(std::integral_constant<bool, false>{});
        alpha_e = alpha;
        // O rescale, only when some lane raised its shift (rare with the lazy max)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
            // in place, so the accumulators keep their registers on both paths;
            // their last writer, the final P.V product of the previous X slot,
            // is more than 64 instructions back
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(acc[db][i]) : "v"(alpha));
        }
    };

    // Prologue: blocks 0-2 into the ring, Q^T into registers.
    for (int t = 0; t < 3 && t < ntiles; ++t) load_block(t);
    pp_barrier<0>();
    if (grp == 1) pp_barrier_lds();

    // X(0)
    if (last_tile >= 0) slot_x(0, std::integral_constant<bool, false>{});
    pp_barrier_lds();
    // Blocks this wave takes part in: Y(t), X(t + 1).  Reads and uses of the
    // operand arrays are unconditional here, so none stays live across the loop.
    for (int t = 0; t <= last_tile; ++t) {
        slot_y(t);
        if (t + 3 < ntiles) load_block(t + 3);
        barrier_y(t);
        slot_x(t + 1, std::integral_constant<bool, true>{});  // after the last block: stale scores, unused
        pp_barrier_lds();
    }
    // Blocks past this wave's rows: loads and barriers only.
    for (int t = last_tile + 1; t < ntiles; ++t) {
        if (t + 3 < ntiles) load_block(t + 3);
        barrier_y(t);
        pp_barrier_lds();
    }
    if (grp == 0) pp_barrier_lds();

    // Epilogue: O = O^T / l per lane (this lane's query), rounded to nearest-even.
    const float l_tot = pair32_sum(l_run);
    const float inv = (l_tot == 0.f) ? 0.f : 1.f / l_tot;
    const int o_rs = (int)(p.o_sr * 2);
    const auto ors = make_rsrc((uint16_t*)p.o + oo + (int64_t)q0 * p.o_sr, (qrows - 1) * o_rs + D * 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + g * 8 + hh * 4;
            uint2 st;
            st.x = Tr::pack2(acc[db][4 * g + 0] * inv, acc[db][4 * g + 1] * inv);
            st.y = Tr::pack2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
            buf_store8(st, ors, lrow * o_rs + d * 2);
        }
    if (hh == 0) {
        const float lse = (l_tot == 0.f) ? kNegInf : (sh_run + fast_log2(l_tot)) * kLn2;
        const auto lrs = make_rsrc(p.lse + lo + q0, qrows * 4);
        buf_store4(lse, lrs, lrow * 4);
    }
}

template <typename Tr, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_prefill_pp(const AttnParams& p, hipStream_t stream) {
    AttnParams q = p;
    q.n_qtiles = (p.L + kPPBlockM - 1) / kPPBlockM;
    const long long grid = (long long)q.n_qtiles * q.Hq * q.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_pp_kernel<Tr, D, CAUSAL, VARLEN>), dim3((unsigned)grid), dim3(512), 0, stream, q);
    return hipGetLastError();
}

}  // namespace sdpa

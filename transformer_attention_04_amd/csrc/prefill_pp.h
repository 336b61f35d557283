// Single-pass attention forward for bf16 / fp16 inputs on gfx950: eight
// wavefronts per workgroup, each owning 32 query rows of a 256-row tile, all
// running the same software-pipelined program over 64-key blocks; one
// resident workgroup per compute unit works through a list of tiles.
//
// Method: the blocked, online-softmax form of exact attention described on the
// khchao.com NN Lab page ("FlashAttention Tiling & Online Softmax Algorithm");
// the result is softmax(scale * Q K^T + mask) V with its logsumexp, as the
// exactref.ai "scaled_dot_product_attention" Full specification defines it.
//
// Schedule.  On gfx950 one wavefront issues a plain vector instruction every
// ~5.7 cycles and an exponential every ~9.3, while a 32x32x16 matrix
// instruction keeps the matrix core busy for 32 cycles; about five vector
// instructions per matrix instruction come for free when two wavefronts share
// a SIMD.  So the softmax of a block is spread between matrix instructions of
// the same wavefront.  Iteration t of a wavefront:
//
//   section 1  S^T(t + 1) = K(t + 1) Q^T (16 products at E = 128) with the
//              softmax of block t between them: row max (lazy shift, raised
//              only when the block max exceeds it by 2^8), then per product
//              four scaled exponentials, then packing of P^T(t) to 16 bits
//   (rare)     O rescale when some lane raised its shift
//   section 2  O^T += V^T(t) P^T(t) (16 products) with the row sum of block t
//              between them
//   end        direct-to-LDS load of one block into the ring, one barrier
//
// Matrix operands are read from LDS six products ahead of their use, in one
// stream (K of block t + 1, then V of block t).  Scores are transposed (one
// query per lane), so P^T is the B operand of the second product without any
// data movement, and Q^T stays in registers for the whole loop.  The vector
// work is pinned in place with empty volatile statements: without them the
// compiler sinks it past the rescale branch into section 2 in one block.
//
// Work list.  Workgroup g takes pairs of tiles (the causal tile with the most
// key blocks and the one with the fewest, so pairs cost alike), pairs g, g + G,
// ...; its key blocks form one stream over all its tiles, so the ring and the
// loads run on across tile boundaries, and the next tile's Q^T is loaded into
// a 64 KB LDS area while the current tile computes.  A tile start then costs
// its first scores only, not the latency of its first loads.
//
// Key and value blocks travel HBM -> LDS by direct-to-LDS buffer loads (no
// staging registers, no LDS write instructions) into a ring of 3 stages:
// waves 0-3 load K blocks three ahead of the compute, waves 4-7 V blocks two
// ahead, each at the end of a step into the stage read one step earlier (K of
// block t + 1 is read in step t, V of block t in step t).  Each lane of a load
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
// The barrier ending step t follows each wave's wait for its older loads (K of
// block t + 2, V of block t + 1: what step t + 1 reads); the load just issued
// may stay in flight.  The first scores of a tile read its K block 0 in the
// tile's first step, so there the barrier precedes the load that refills it.
// Buffer resources turn reads past the last key into zeros; keys past the
// last key or past the causal diagonal get the score -inf (edge blocks only).
//
// Float mask (MASK_FLOAT).  The logit is one fp32 FMA, scale * s + bias, and
// the shift and exponentials then work on logits (factor log2 e instead of
// scale * log2 e), so any scale works.  Each wave moves the bias of its own 32
// rows for one key block (8 KB) by direct-to-LDS loads into its own 8 KB of
// LDS, one block ahead of use: the load is issued right after the wave has
// read the previous block's bias, and the bias of block t + 1 is read and
// added to the scores of block t + 1 in section 2 of iteration t (the first
// block's at the start of its tile).  Each load moves four whole 256-byte
// rows; chunk c of row r sits at position c ^ (r mod 16) of the row, so the
// 16-byte reads of 16 rows fall in distinct banks.  The 64 KB this takes
// come from the Q^T staging area: Q^T is loaded into registers at each tile
// start instead.  Causal and edge masking are applied after the bias.
//
// Paged key/value cache (PAGED; chunked prefill: the L new rows of each
// sequence are its last L positions, causal aligned bottom-right): the key
// blocks of sequence b are read through its row of the block table.  The
// direct-to-LDS loads of one wave and block cover exactly one 16-key group
// (rows 16w .. 16w + 15 of wave w of either group), which lies inside one
// page (pages hold a power of two >= 16 keys), so each wave looks up one page
// per block: the table row of the cursor's sequence sits in the wave's lanes
// (loaded when the cursor enters a new sequence) and the group's entry comes
// out with readlane.  An entry outside the pool is never dereferenced: its K
// rows come from a block of NaN rows and its V rows read as 0, so exactly the
// rows that keep one of its keys come out NaN.  Pool rows must be contiguous
// (row stride E) for that NaN block's layout to match.  With VARQ the new
// rows of sequence b are packed at tokens cu_q[b] .. (their own count, at
// most L); tiles past a sequence's rows are items with no rows, which take
// one step of the ring and compute nothing.
//
// Bool mask (MASK_BOOL; rows in whole 16-byte chunks, positive scale): the
// same cursor moves the wave's 32 rows x 64 keys of mask bytes (2 KB) in two
// direct-to-LDS loads per block; each lane reads 8 bytes per 16-key chunk
// (conflict-free: a load's lane order puts row r's chunk c at (16c + r%16) *
// 16) and sets the scores of masked keys to -inf before the row maximum.
#pragma once

#include "attn_common.h"
#include "device_utils.h"

#include <type_traits>
#include <utility>

namespace sdpa {

constexpr int kPPBlockM = 256;  // query rows per workgroup

// Calls f(integral_constant<int, i>) for i = 0 .. N-1 (compile-time indices).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Swap bits 2 and 3 of a key index within its 32-key block.
__device__ __forceinline__ int swap_bits23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Exponent margin (log2 units) by which a block max may exceed the current
// shift before the shift is raised.
constexpr float kLazyRescale = 8.0f;

// End of a step: this wave's LDS accesses, and all but VM of its direct-to-LDS
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

// pp_barrier<vm> for a wave-uniform vm taken from {0, A, B, A + B} (the counts
// the first item's waits use).
template <int A, int B>
__device__ __forceinline__ void pp_barrier_of(int vm) {
    if (vm == A + B)
        pp_barrier<A + B>();
    else if (vm == B)
        pp_barrier<B>();
    else if (vm == A)
        pp_barrier<A>();
    else
        pp_barrier<0>();
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

// max of three floats in one instruction, without the quieting copies the
// compiler adds in front of fmaxf on values it cannot prove canonical (a NaN
// score makes its row NaN through the exponentials either way).  Only used on
// scores produced by matrix instructions of the previous iteration.
__device__ __forceinline__ float pp_max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Pins a value's computation to this point of the instruction stream.  Without
// it, code motion after scheduling sinks work into the block that first uses
// it (past the branch of the rare O rescale, or past a barrier), which would
// undo the interleaving of vector work with matrix instructions.
__device__ __forceinline__ void pp_pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pp_pin(uint32_t& x) { asm volatile("" : "+v"(x)); }

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

// Work of one workgroup: pairs of 256-row query tiles of one (batch, head),
// the tile with the most key blocks together with the one with the fewest
// (tiles nq - 1 - i and i), so that every pair costs about the same under the
// causal mask.  Workgroup g takes pairs g, g + G, g + 2G, ... (G workgroups,
// at most one per compute unit, all resident at once); workgroups are dealt to
// the 8 XCDs round-robin, so pair P runs on XCD P % 8 when G is a multiple of
// 8, and the numbering of pp_pair keeps the tiles of a head on one XCD and in
// flight together.
struct PPWork {
    int nbh;       // batch * heads
    int nq;        // query tiles per head
    int n_pairs;   // nbh * ceil(nq / 2)
    int xcd;       // 1: pairs numbered by XCD (see pp_pair below), 0: head-major
    int npp_log2;  // by XCD: log2 of the pairs per head, ceil(nq / 2)
    int b_log2;    // by XCD: log2 of the batch size
};

// Head (b * Hq + h) and pair index within the head of pair P.  Head-major:
// P = pp * nbh + bh.  By XCD (when Hq and the grid are multiples of 8 and the
// pairs per head and the batch size are powers of two, so that no division is
// needed): the
// pairs of XCD x = P % 8 (where workgroups g = x + 8k run) are numbered t = P / 8
// in the order they run there, the ceil(nq / 2) pairs of one head consecutive
// and the B heads that share a head index h next to each other, so that all
// tiles of a (b, h) run on one XCD at the same time (sharing its K/V in L2)
// and so do the B batches of a head (sharing a mask broadcast over the batch).
// XCD x takes the heads h = x mod 8, or with CONTIG (paged caches, where
// grouped query heads are the rule) the contiguous heads x Hq / 8 ..
// (x + 1) Hq / 8 - 1, so that the query heads of a key/value group read its
// pages through one L2.
template <bool CONTIG = false>
__device__ __forceinline__ void pp_pair(const PPWork& w, int B, int Hq, int P, int& bh, int& pp) {
    if (w.xcd) {
        const int x = P & 7, t = P >> 3;
        const int u = t >> w.npp_log2;
        pp = t & ((1 << w.npp_log2) - 1);
        const int b = u & ((1 << w.b_log2) - 1), m = u >> w.b_log2;
        bh = CONTIG ? b * Hq + x * (Hq >> 3) + m : b * Hq + m * 8 + x;
    } else {
        bh = P % w.nbh;
        pp = P / w.nbh;
    }
}

// 16 key rows of all-ones 16-bit words (NaN in bf16 and fp16) at the widest
// head dim: the K rows a paged call reads for a block-table entry outside the
// page pool, so that exactly the rows that keep one of its keys come out NaN.
struct PPNanRows {
    uint32_t w[16 * 128 / 2];
};
constexpr PPNanRows pp_make_nan_rows() {
    PPNanRows x{};
    for (int i = 0; i < 16 * 128 / 2; ++i) x.w[i] = 0xffffffffu;
    return x;
}
static __device__ const PPNanRows kPPNanRows = pp_make_nan_rows();

template <typename Tr, int D, bool CAUSAL, int MASK = MASK_NONE, bool PAGED = false, bool VARQ = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_pp_kernel(AttnParams p, PPWork w) {
    constexpr bool FMASK = MASK == MASK_FLOAT;
    constexpr bool BMASK = MASK == MASK_BOOL;
    constexpr bool ANYMASK = FMASK || BMASK;
    constexpr int BM = kPPBlockM;
    constexpr int BN = 64;
    constexpr int NC = D / 8;          // 16-byte chunks per row
    constexpr int KTILE = BN * D;      // one K or V block, 16-bit words
    constexpr int NSTAGE = 3;          // ring of K/V stages
    constexpr int STAGE = 2 * KTILE;   // K block then V block
    constexpr int QAREA = ANYMASK ? 0 : BM * D;   // Q^T of the next tile, 16-bit words
    // mask of one block per wave (fp32 bias or bool bytes), 16-bit words
    constexpr int MBYTES = FMASK ? 4 : 1;                 // bytes per mask element
    constexpr int WAREA = 32 * BN * MBYTES;               // bytes per wave
    constexpr int BAREA = ANYMASK ? 8 * WAREA / 2 : 0;
    constexpr int NKK = D / 16;        // k-steps of the score product
    constexpr int NDB = D / 32;        // 32-row blocks of O^T
    constexpr int NDMA = NC / 4;       // direct-to-LDS loads per wave per block
    constexpr int NQDMA = NC / 2;      // direct-to-LDS loads per wave per Q tile
    constexpr int NBDMA = BMASK ? 2 : 8;   // direct-to-LDS loads per wave per mask block
    constexpr int NBRD = BMASK ? 4 : 8;    // mask reads per lane per block
    static_assert(D == 64 || D == 96 || D == 128, "head dim must be 64, 96 or 128");
    static_assert(!(PAGED && MASK != MASK_NONE), "no mask on a paged cache");
    static_assert(!VARQ || PAGED, "packed query rows only against a paged cache");
    static_assert(2 * NKK == 4 * NDB, "one K operand read per P.V product");
    static_assert((NSTAGE * STAGE + QAREA + BAREA) * 2 <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) uint16_t smem[NSTAGE * STAGE + QAREA + BAREA];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int grp = wave >> 2;     // 0: loads K, 1: loads V
    const int wg = wave & 3;
    const int lq = lane & 31;
    const int hh = lane >> 5;
    const int G = (int)gridDim.x;
    const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

    // Items of this workgroup: (pair P, half s); s = 0 is the tile with more
    // key blocks.  A pair whose two tiles coincide (odd nq) has one item.
    auto pair_qt = [&](int P, int s) {
        int bh, pp;
        pp_pair<PAGED>(w, p.B, p.Hq, P, bh, pp);
        return s == 0 ? w.nq - 1 - pp : pp;
    };
    auto next_item = [&](int& P, int& s) {
        int bh, pp;
        pp_pair<PAGED>(w, p.B, p.Hq, P, bh, pp);
        if (s == 0 && w.nq - 1 - pp != pp) {
            s = 1;
        } else {
            P += G;
            s = 0;
        }
    };
    // Key blocks of tile qt (at least one, so that every item takes one step
    // of the ring; an empty causal range gives a block of zeros and no work).
    // sk: the keys of the item's sequence (p.S, or on a paged cache the
    // sequence's own count, its L query rows being its last L positions:
    // causal aligns bottom-right).
    auto seq_keys = [&](int b) {
        if constexpr (PAGED)
            return min(max(p.seq_lens[b], 0), min(p.S, p.max_blocks << p.page_shift));
        else
            return p.S;
    };
    // VARQ (packed new rows of each sequence, tokens cu_q[b] ..): the rows of
    // sequence b and its first token; tiles past its rows are empty items
    auto seq_tok0 = [&](int b) -> int64_t {
        if constexpr (VARQ)
            return min(max((int64_t)p.cu_q[b], (int64_t)0), p.total_q);
        else
            return 0;
    };
    auto seq_rows = [&](int b) {
        if constexpr (VARQ) {
            const int64_t a = seq_tok0(b);
            return (int)min(min(max((int64_t)p.cu_q[b + 1], a), p.total_q) - a, (int64_t)p.L);
        } else {
            return p.L;
        }
    };
    auto kend_of = [&](int qt, int sk, int lq) {
        if constexpr (PAGED) {
            if (VARQ && qt * BM >= lq) return 0;
            return CAUSAL ? max(0, min(sk, min(qt * BM + BM, lq) + sk - lq)) : sk;
        } else {
            return CAUSAL ? min(sk, min(qt * BM + BM, lq)) : sk;
        }
    };
    auto steps_of = [&](int qt, int sk, int lq) { return max(1, (kend_of(qt, sk, lq) + BN - 1) / BN); };
    auto head_of = [&](int P, int& b, int& h, int& kvh) {
        int bh, pp;
        pp_pair<PAGED>(w, p.B, p.Hq, P, bh, pp);
        h = bh % p.Hq;
        b = bh / p.Hq;
        kvh = h / p.group;
    };

    // Direct-to-LDS loads of a K/V block: waves 0-3 move K, waves 4-7 move V,
    // NDMA loads of 64 chunks per wave.  g_off[i] is the global byte offset
    // (within the block) of the chunk this lane places for load i.
    const int k_rs = (int)(p.k_sr * 2);
    const int v_rs = (int)(p.v_sr * 2);
    int g_off[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        const int P = (wg * NDMA + i) * 64 + lane;  // LDS chunk position in the block
        if (grp == 0) {
            const int r = (P / (16 * NC)) * 16 + P % 16, c = (P % (16 * NC)) / 16;
            const int row = (r & ~31) | swap_bits23(r & 31);
            g_off[i] = (row - (PAGED ? 16 * wg : 0)) * k_rs + c * 16;
        } else {
            const int k = (P / (4 * NC)) * 4 + P % 4, c = (P % (4 * NC)) / 4;
            g_off[i] = (k - (PAGED ? 16 * wg : 0)) * v_rs + c * 16;
        }
    }
    const int g_rs = grp == 0 ? k_rs : v_rs;
    const int64_t g_sr = grp == 0 ? p.k_sr : p.v_sr;
    const int64_t g_sb = grp == 0 ? p.k_sb : p.v_sb;
    const int64_t g_sh = grp == 0 ? p.k_sh : p.v_sh;
    const uint16_t* g_ptr = (const uint16_t*)(grp == 0 ? p.k : p.v);

    // The load cursor of a wave walks the workgroup's key blocks in processing
    // order (all items, every block of each): waves 0-3 move K blocks three
    // ahead of the compute, waves 4-7 V blocks two ahead.  Returns whether a
    // load was issued.
    // Per-item quantities (head pointer, block count) are set when the cursor
    // enters an item; a block costs a few scalar instructions.
    // Paged cache: each wave's part of a block is one 16-key group (rows 16wg
    // .. 16wg + 15), which lies inside one page; the cursor keeps the block
    // table row of its sequence in the wave's lanes (entry 64j + lane in
    // ltab[j], at most 256 pages) and takes the group's page with readlane.
    int lP = (int)blockIdx.x, ls = 0, lt = 0, lsteps = 0, lstage = 0;
    const uint16_t* lptr = g_ptr;  // K or V of the cursor's head, at block lt (paged: the pool's head)
    int lS = p.S, lb = -1;         // paged: keys and index of the cursor's sequence
    int lL = p.L;                  // its query rows
    int ltab[PAGED ? 4 : 1];
    auto load_enter = [&] {
        if (lP < w.n_pairs) {
            int b, h, kvh;
            head_of(lP, b, h, kvh);
            if constexpr (PAGED) {
                lptr = g_ptr + (int64_t)kvh * g_sh;
                if (b != lb) {
                    lb = b;
                    lS = seq_keys(b);
                    lL = seq_rows(b);
                    const auto tr = make_rsrc(p.block_table + (int64_t)b * p.bt_stride, p.max_blocks * 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) ltab[j] = (int)buf_load4(tr, (j * 64 + lane) * 4);
                }
            } else {
                lptr = g_ptr + (int64_t)b * g_sb + (int64_t)kvh * g_sh;
            }
            lsteps = steps_of(pair_qt(lP, ls), lS, lL);
        }
    };
    load_enter();
    auto load_next = [&] {
        if (lP >= w.n_pairs) return false;
        u32x4_t rs;
        if constexpr (PAGED) {
            const int k16 = lt * BN + 16 * wg;
            const int nv = min(16, lS - k16);
            int pg = -1;
            if (nv > 0) {
                const int ix = k16 >> p.page_shift, j = ix >> 6, ln = ix & 63;
                pg = j == 0 ? __builtin_amdgcn_readlane(ltab[0], ln)
                   : j == 1 ? __builtin_amdgcn_readlane(ltab[1], ln)
                   : j == 2 ? __builtin_amdgcn_readlane(ltab[2], ln)
                            : __builtin_amdgcn_readlane(ltab[3], ln);
            }
            const bool ok = nv > 0 && (unsigned)pg < (unsigned)p.n_pages;
            // a kept key on a page outside the pool: K rows of NaN, V rows of 0
            const uint16_t* src = ok ? lptr + (int64_t)pg * g_sb + (int64_t)(k16 & ((1 << p.page_shift) - 1)) * g_sr
                                     : (const uint16_t*)kPPNanRows.w;
            rs = pp_rsrc(src, (ok || (nv > 0 && grp == 0)) ? (nv - 1) * g_rs + D * 2 : 0);
        } else {
            const int rows = min(BN, p.S - lt * BN);
            rs = pp_rsrc(lptr, (rows - 1) * g_rs + D * 2);
        }
        const uint32_t dst = smem_addr + (uint32_t)((lstage * STAGE + grp * KTILE) * 2 + wg * NDMA * 1024);
#pragma unroll
        for (int i = 0; i < NDMA; ++i) pp_dma16(rs, g_off[i], dst + i * 1024);
        lstage = lstage == NSTAGE - 1 ? 0 : lstage + 1;
        if constexpr (!PAGED) lptr += (int64_t)BN * g_sr;
        if (++lt == lsteps) {
            next_item(lP, ls);
            lt = 0;
            load_enter();
        }
        return true;
    };

    // Q^T of a tile: each wave moves its own 32 rows into its own part of the
    // Q area (chunk layout as for K), so it alone reads them and no barrier
    // guards the area.
    const uint32_t q_lds = smem_addr + (uint32_t)((NSTAGE * STAGE + wave * 32 * D) * 2);
    const int q_rs = (int)(p.q_sr * 2);
    auto load_q = [&](int P, int s) {
        int b, h, kvh;
        head_of(P, b, h, kvh);
        const int q0 = pair_qt(P, s) * BM;
        const int rows = min(32, seq_rows(b) - q0 - wave * 32);
        const int64_t qoff = VARQ ? (int64_t)h * p.q_sh + (seq_tok0(b) + q0 + wave * 32) * p.q_sr
                                  : (int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)(q0 + wave * 32) * p.q_sr;
        const u32x4_t rs = pp_rsrc((const uint16_t*)p.q + qoff, (rows - 1) * q_rs + D * 2);
        // lane index made opaque here, so that the per-lane offsets below are
        // computed per tile and not kept in registers across the whole loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < NQDMA; ++i) {
            const int P2 = i * 64 + ln;
            const int r = (P2 / (16 * NC)) * 16 + P2 % 16, c = (P2 % (16 * NC)) / 16;
            pp_dma16(rs, r * q_rs + c * 16, q_lds + i * 1024);
        }
    };

    // Float mask: a second cursor walks the blocks this wave computes (all
    // items, block 0 .. last of each; items where the wave has no rows are
    // skipped) and loads the bias of one block into the wave's 8 KB area.
    // Load i, lane m: row 4i + m/16 of the wave's 32, chunk (m%16) ^ (row%16)
    // of the row's 16 chunks of 4 keys; relative to row 16(i/4), the lane's
    // byte offset depends on i only through i%4.
    // Bool mask: the same cursor moves 32 rows x 64 bytes per block in two
    // loads; load i, lane m: row 16i + m%16, 16-byte chunk m/16 (keys
    // 16(m/16) .. +15), so the chunk a lane reads sits at (chunk*16 + row%16)*16.
    const uint32_t b_lds = smem_addr + (uint32_t)((NSTAGE * STAGE + QAREA) * 2 + wave * WAREA);
    const int m_rs = (int)(p.m_sr * MBYTES);
    int b_off[4];
    if constexpr (FMASK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * i + (lane >> 4);
            b_off[i] = row * m_rs + (((lane & 15) ^ (row & 15)) * 16);
        }
    } else if constexpr (BMASK) {
        b_off[0] = b_off[1] = b_off[2] = b_off[3] = (lane & 15) * m_rs + (lane >> 4) * 16;
    }
    int bP = (int)blockIdx.x, bs = 0, bt = 0, blast = -1;
    using MElem = std::conditional_t<FMASK, float, uint8_t>;
    const MElem* bptr = (const MElem*)p.mask;  // mask of the cursor's item, first row of this wave
    int brows = 0;                              // rows of this wave in that item
    auto bias_enter = [&] {
        while (bP < w.n_pairs) {
            int b, h, kvh;
            head_of(bP, b, h, kvh);
            const int qt = pair_qt(bP, bs);
            const int qrows = min(BM, p.L - qt * BM);
            const int ntl = (kend_of(qt, p.S, p.L) + BN - 1) / BN;
            blast = wave * 32 >= qrows ? -1
                    : CAUSAL ? min(ntl - 1, (qt * BM + wave * 32 + 31) / BN)
                             : ntl - 1;
            if (blast >= 0) {
                brows = min(32, qrows - wave * 32);
                bptr = (const MElem*)p.mask + (int64_t)b * p.m_sb + (int64_t)h * p.m_sh +
                       (int64_t)(qt * BM + wave * 32) * p.m_sr;
                return;
            }
            next_item(bP, bs);
        }
    };
    // Issues the cursor's block (NBDMA loads) and advances; false when no block
    // is left.  Rows 0-15 and 16-31 get a buffer resource each, whose base is
    // their first row at the block's first key and whose size ends at the last
    // key of the wave's last row, so every byte read is range checked.
    auto bias_next = [&] {
        if (bP >= w.n_pairs) return false;
        const MElem* base = bptr + bt * BN;
        const int kbytes = (p.S - bt * BN) * MBYTES;
        const u32x4_t rs0 = pp_rsrc(base, (brows - 1) * m_rs + kbytes);
        const u32x4_t rs1 = pp_rsrc((const char*)base + (int64_t)16 * m_rs, (brows - 17) * m_rs + kbytes);
#pragma unroll
        for (int i = 0; i < NBDMA; ++i)
            pp_dma16(i < NBDMA / 2 ? rs0 : rs1, b_off[i & 3], b_lds + i * 1024);
        if (++bt > blast) {
            next_item(bP, bs);
            bt = 0;
            bias_enter();
        }
        return true;
    };
    // Bias reads: lane (lq, hh), read i = (kb, c, half) -> keys kb*32 + c*16 +
    // 8hh + 4half + 0..3 of row lq, i.e. chunk J + 2hh with J = 8kb + 4c + half;
    // its position (J + 2hh) ^ (lq % 16) = J ^ z is one XOR away from a lane base.
    // (byte offsets from smem; the area and each row are 256-byte aligned, so
    // the XOR only touches bits 4-7)
    int b_rd = 0;
    if constexpr (FMASK) {
        const int z = (2 * hh) ^ (lq & 15);
        b_rd = ((NSTAGE * STAGE + QAREA) * 2 + wave * WAREA + lq * 256) ^ (z * 16);
    } else if constexpr (BMASK) {
        // read i = (kb, c): keys 16(2kb + c) + 8hh + 0..7 of row lq
        b_rd = (NSTAGE * STAGE + QAREA) * 2 + wave * WAREA + (lq >> 4) * 1024 + (lq & 15) * 16 + hh * 8;
    }
    auto bias_read = [&](int i) {
        if constexpr (BMASK) {
            return *(const uint2*)((const char*)smem + b_rd + i * 256);
        } else {
            const int J = 8 * (i >> 2) + 4 * ((i >> 1) & 1) + (i & 1);
            return *(const float4*)((const char*)smem + (b_rd ^ (J * 16)));
        }
    };
    // Adds bias read i (4 keys) to the scores: logit = |scale| * s + bias.
    // Bool mask: read i (8 bytes) decides scores s[kb][8c + 0..7], kb = i/2, c = i%2.
    auto mask_apply = [&](f32x16_t* s, int i, uint2 bv) {
        const int kb = i >> 1, r0 = (i & 1) * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t byte = ((r < 4 ? bv.x : bv.y) >> (8 * (r & 3))) & 0xffu;
            float l = byte != 0 ? s[kb][r0 + r] : kNegInf;
            pp_pin(l);
            s[kb][r0 + r] = l;
        }
    };
    auto bias_add = [&](f32x16_t* s, int i, auto bv) {
        if constexpr (BMASK) {
            mask_apply(s, i, bv);
        } else {
            const int kb = i >> 2, r0 = ((i >> 1) & 1) * 8 + (i & 1) * 4;
            float l[4] = {fmaf(s[kb][r0 + 0], p.scale_abs, bv.x), fmaf(s[kb][r0 + 1], p.scale_abs, bv.y),
                          fmaf(s[kb][r0 + 2], p.scale_abs, bv.z), fmaf(s[kb][r0 + 3], p.scale_abs, bv.w)};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pp_pin(l[r]);
                s[kb][r0 + r] = l[r];
            }
        }
    };
    using MaskRead = std::conditional_t<BMASK, uint2, float4>;
    bool kv_after_bias = false;  // direct-to-LDS K/V loads were issued after the latest bias load

    // K operand: LDS row kb*32 + lq, chunk kk*2 + hh -> position
    // (row/16)*16*NC + chunk*16 + row%16.  The Q area uses the same layout.
    const int k_lane = ((lq >> 4) * 16 * NC + hh * 16 + (lq & 15)) * 16;  // bytes
    // V^T operand of chunk ch (keys ch*16 + 8hh + 0..7), rows db*32 + 0..31:
    // two transposing reads of 4 keys each.  Lane i of a 16-lane group reads
    // key k0 + i/4, columns d0 + 4(i%4) .. +3, where d0 = db*32 + 16*(lane/16 & 1).
    const int vi = lane & 15;
    const int v_lane = ((hh * 2) * 4 * NC + (2 * ((lane >> 4) & 1) + (vi & 3) / 2) * 4 + vi / 4) * 16 + (vi & 1) * 8;

    uint4 qreg[NKK];  // Q^T operand of the current tile
    f32x16_t acc[NDB];
    float sh_run;     // running shift, log2 units (-inf until a kept key)
    float l_run;      // this lane's share of the row sum relative to it (fp32 weights, for lse)
    float lr_run;     // the same over the weights rounded to 16 bits (normalises the output)
    const float cfac = FMASK ? kLog2e : p.scale_log2;  // log2-domain factor of a score (or logit)
    f32x16_t sA[2], sB[2];   // scores of block t and t + 1, roles swapping each iteration
    // current item
    int Sb = p.S, q0 = 0, wrow0 = wave * 32, my_row = 0;
    int coff = 0;   // paged: keys before the first query row (causal aligns bottom-right)

    typedef short s16x4 __attribute__((ext_vector_type(4)));
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // V^T operand j = (chunk ch, 32 rows db) of the block in stage st: keys
    // ch*16 + 8hh + 0..7, two transposing reads of 4 keys each.
    auto read_v = [&](int st, int j) {
        const int ch = j / NDB, db = j % NDB;
        const char* Vb = (const char*)(smem + st * STAGE + KTILE) + v_lane;
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
    auto read_k = [&](int st, int i) {  // K operand i = (kk = i/2, kb = i%2) of the block in stage st
        const char* Kb = (const char*)(smem + st * STAGE) + k_lane;
        return *(const uint4*)(Kb + ((i & 1) * 2 * 16 * NC + (i >> 1) * 2 * 16) * 16);
    };
    constexpr int NOP = 2 * NKK;  // products per half (16 at E = 128)
    static_assert(NOP == 4 * NDB, "one K operand read per P.V product");
    constexpr int LA = 6;         // operand reads run this many products ahead

    // S^T = K Q^T of the block in stage st into s_out, operands streamed from LDS.
    auto scores = [&](int st, f32x16_t* s_out) {
        uint4 kop[NOP];
#pragma unroll
        for (int j = 0; j < LA; ++j) kop[j] = read_k(st, j);
        fence();
#pragma unroll
        for (int j = 0; j < NOP; ++j) {
            if (j + LA < NOP) kop[j + LA] = read_k(st, j + LA);
            fence();
            s_out[j & 1] = Tr::mfma32(as_vec8<Tr>(kop[j]), as_vec8<Tr>(qreg[j >> 1]), j < 2 ? f32x16_t{} : s_out[j & 1]);
            fence();
        }
    };

    // Scores of keys outside the block's kept range (past the last key, or past
    // the causal diagonal) become -inf in place; their weights then come out
    // as exp2(-inf) = 0 (the scale is positive here).
    auto mask_scores = [&](int t, f32x16_t* s_cur) {
        const int key0 = t * BN;
        // s_cur[kb][8c + j] is the score of key key0 + 32kb + 16c + 8hh + j for query my_row.
        int lim = Sb - (key0 + hh * 8);
        if (CAUSAL) lim = min(lim, my_row + 1 + coff - (key0 + hh * 8));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int li = kb * 32 + (r >> 3) * 16 + (r & 7);
                s_cur[kb][r] = li < lim ? s_cur[kb][r] : kNegInf;
            }
    };

    // One iteration for block t (its K/V in stage stc, the next block's in stn):
    // the scores of block t + 1 on the matrix core with the softmax of block t
    // between the products, then O^T += V^T P^T of block t with its row sum
    // between the products.
    auto iteration = [&](int stc, int stn, f32x16_t* s_cur, f32x16_t* s_next) {
        uint4 pb[4];
        float m4[4];
        float alpha = 1.f, shift = 0.f;
        // the 16 steps of the softmax, one after each score product (E = 128;
        // smaller head dims run several steps per product)
        auto soft_step = [&](auto step_tag) {
            constexpr int st = decltype(step_tag)::value;
            if constexpr (st < 4) {
                const int kb = st >> 1, r0 = (st & 1) * 8;
                const float a = pp_max3(s_cur[kb][r0 + 0], s_cur[kb][r0 + 1], s_cur[kb][r0 + 2]);
                const float b = pp_max3(s_cur[kb][r0 + 3], s_cur[kb][r0 + 4], s_cur[kb][r0 + 5]);
                m4[st] = pp_max3(a, b, pp_max3(s_cur[kb][r0 + 6], s_cur[kb][r0 + 7], s_cur[kb][r0 + 7]));
            } else if constexpr (st == 4) {
                float mx = pp_max3(pp_max3(m4[0], m4[1], m4[2]), m4[3], m4[3]);
                mx = pair32_max(mx);
                const float mxs = mx * cfac;
                const bool raise = mxs > sh_run + kLazyRescale;
                const float sh_new = raise ? mxs : sh_run;
                alpha = raise ? fast_exp2(sh_run - sh_new) : 1.f;
                sh_run = sh_new;
                shift = (sh_new == kNegInf) ? 0.f : sh_new;
            } else if constexpr (st < 13) {
                // four weights per step, in place
                const int base = (st - 5) * 4, kb = base >> 4, r0 = base & 15;
#pragma unroll
                for (int r = r0; r < r0 + 4; ++r) s_cur[kb][r] = fmaf(s_cur[kb][r], cfac, -shift);
#pragma unroll
                for (int r = r0; r < r0 + 4; ++r) {
                    float e = fast_exp2(s_cur[kb][r]);
                    pp_pin(e);
                    s_cur[kb][r] = e;
                }
            } else {
                // pack P^T: steps 13, 14, 15 cover chunks 0-1, 2, 3
#pragma unroll
                for (int q = (st == 13 ? 0 : st - 12); q <= (st == 13 ? 1 : st - 12); ++q) {
                    const int kb = q >> 1, c = q & 1;
                    uint4 u;
                    u.x = Tr::pack2(s_cur[kb][c * 8 + 0], s_cur[kb][c * 8 + 1]);
                    u.y = Tr::pack2(s_cur[kb][c * 8 + 2], s_cur[kb][c * 8 + 3]);
                    u.z = Tr::pack2(s_cur[kb][c * 8 + 4], s_cur[kb][c * 8 + 5]);
                    u.w = Tr::pack2(s_cur[kb][c * 8 + 6], s_cur[kb][c * 8 + 7]);
                    pp_pin(u.x);
                    pp_pin(u.y);
                    pp_pin(u.z);
                    pp_pin(u.w);
                    pb[q] = u;
                }
            }
        };
        // One stream of 2 NOP operand reads per iteration, LA ahead of use: the
        // K operands of block t + 1 (score products), then the V^T operands of
        // block t (P.V products).  The first reads are covered by the row-max
        // steps of the softmax, which do not wait for them.
        uint4 opq[2 * NOP];
        auto issue = [&](auto it) {
            constexpr int i = decltype(it)::value;
            if constexpr (i < NOP)
                opq[i] = read_k(stn, i);
            else if constexpr (i < 2 * NOP)
                opq[i] = read_v(stc, i - NOP);
        };
        static_for<LA>([&](auto it) { issue(it); });
        fence();
        static_for<4>([&](auto st) { soft_step(st); });
        fence();
        // section 1: score products of block t + 1, softmax steps 4-15 of block t between them
        static_for<NOP>([&](auto jt) {
            constexpr int j = decltype(jt)::value;
            issue(std::integral_constant<int, j + LA>{});
            fence();
            // the first product of each chain starts from the constant 0
            s_next[j & 1] = Tr::mfma32(as_vec8<Tr>(opq[j]), as_vec8<Tr>(qreg[j >> 1]), j < 2 ? f32x16_t{} : s_next[j & 1]);
            static_for<(12 * (j + 1)) / NOP - (12 * j) / NOP>([&](auto kt) {
                soft_step(std::integral_constant<int, 4 + (12 * j) / NOP + decltype(kt)::value>{});
            });
            fence();
        });
        // O rescale, only when some lane raised its shift (rare with the lazy max)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
            // in place, so the accumulators keep their registers on both paths;
            // their last writer, the final P.V product of the previous
            // iteration, is more than 16 matrix instructions back
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(acc[db][i]) : "v"(alpha));
        }
        fence();
        // section 2: O^T += V^T P^T of block t, row sum between the products;
        // masks: the bias (or bool mask) of block t + 1 applied to its scores
        // between the last NBRD products (the wait for its load at the first)
        {
            float p8[8], r4[4];
            MaskRead bq;
            static_for<NOP>([&](auto jt) {
                constexpr int j = decltype(jt)::value;
                issue(std::integral_constant<int, NOP + j + LA>{});
                fence();
                acc[j % NDB] = Tr::mfma32(as_vec8<Tr>(opq[NOP + j]), as_vec8<Tr>(pb[j / NDB]), acc[j % NDB]);
                // row-sum items [13 j / NOP, 13 (j + 1) / NOP): 8 partial sums of the fp32
                // weights, 4 of the rounded ones (the P^T operand chunks), and the updates
                static_for<(13 * (j + 1)) / NOP - (13 * j) / NOP>([&](auto it) {
                    constexpr int w = (13 * j) / NOP + decltype(it)::value;
                    if constexpr (w < 8) {
                        p8[w] = (s_cur[w >> 2][(w & 3) * 4 + 0] + s_cur[w >> 2][(w & 3) * 4 + 1]) +
                                (s_cur[w >> 2][(w & 3) * 4 + 2] + s_cur[w >> 2][(w & 3) * 4 + 3]);
                        pp_pin(p8[w]);
                    } else if constexpr (w < 12) {
                        const uint4 u = pb[w - 8];
                        r4[w - 8] = Tr::sum2(u.w, Tr::sum2(u.z, Tr::sum2(u.y, Tr::sum2(u.x, 0.f))));
                        pp_pin(r4[w - 8]);
                    } else {
                        const float tsum = ((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]));
                        l_run = fmaf(l_run, alpha, tsum);
                        lr_run = fmaf(lr_run, alpha, (r4[0] + r4[1]) + (r4[2] + r4[3]));
                        pp_pin(l_run);
                        pp_pin(lr_run);
                    }
                });
                if constexpr (ANYMASK) {
                    constexpr int J0 = NOP - NBRD;
                    if constexpr (j == J0) {
                        // read addresses computed here, not kept in registers across the loop
                        asm volatile("" : "+v"(b_rd));
                        // vmcnt only (lgkmcnt left at its maximum: operand reads stay in flight)
                        if (kv_after_bias)
                            __builtin_amdgcn_s_waitcnt(0x0F70 | NDMA);
                        else
                            __builtin_amdgcn_s_waitcnt(0x0F70);
                        bq = bias_read(0);
                    } else if constexpr (j > J0) {
                        const MaskRead cv = bq;
                        bq = bias_read(j - J0);
                        bias_add(s_next, j - J0 - 1, cv);
                    }
                }
                fence();
            });
            if constexpr (ANYMASK) bias_add(s_next, NBRD - 1, bq);
        }
    };

    // Prologue: Q^T of the first item (float mask: the bias of the wave's
    // first block instead), K blocks 0-2 and V blocks 0-1.
    // Without a mask the first scores need only Q^T and K block 0: the barrier
    // waits for those, and K blocks 1-2 (K waves) and V blocks 0-1 (V waves) land
    // during the first scores (a second barrier before the first step's
    // products waits for K block 1 and V block 0).  vmcnt counts the loads in
    // the order they were issued.
    int P = (int)blockIdx.x, s = 0;
    int n_kv = 0;  // K or V blocks this wave loaded in the prologue
    if constexpr (ANYMASK) {
        bias_enter();
        bias_next();
    } else {
        load_q(P, 0);
    }
    for (int i = 0; i < 3 - grp; ++i) n_kv += load_next() ? 1 : 0;
    if constexpr (ANYMASK) {
        pp_barrier<0>();
    } else {
        const int later = grp == 0 ? max(n_kv - 1, 0) : n_kv;  // blocks allowed in flight
        pp_barrier_of<NDMA, 2 * NDMA>(later * NDMA);
    }
    bool first_item = true;
    int cur = 0;  // ring stage of the current block
    auto advance = [](int st) { return st == NSTAGE - 1 ? 0 : st + 1; };

    while (P < w.n_pairs) {
        int b, h, kvh;
        head_of(P, b, h, kvh);
        q0 = pair_qt(P, s) * BM;
        my_row = q0 + wrow0 + lq;
        const int Lb = seq_rows(b);
        const int64_t tok0 = seq_tok0(b);
        if constexpr (PAGED) {
            Sb = seq_keys(b);
            coff = Sb - Lb;
        }
        const int ntiles = (kend_of(q0 / BM, Sb, Lb) + BN - 1) / BN;  // 0 when no key is kept
        const int nsteps = max(1, ntiles);
        const int qrows = min(BM, Lb - q0);
        const bool wave_has_rows = wrow0 < qrows;
        // last key block this wave takes part in (causal: its last row's block)
        const int last_tile = !wave_has_rows ? -1
                              : CAUSAL ? min(ntiles - 1, (q0 + wrow0 + 31 + coff) / BN)
                                       : ntiles - 1;
        int nP = P, ns = s;
        next_item(nP, ns);
        const bool has_next = nP < w.n_pairs;

        // Q^T from this wave's part of the Q area (every barrier so far waited
        // for all of the wave's loads), or (float mask) straight from memory:
        // lane (lq, hh) holds elements 16kk + 8hh .. +7 of its row.  Negated
        // when the scale is negative.
        if constexpr (ANYMASK) {
            const int q_rows = max(0, min(32, qrows - wrow0));
            const auto qrs = make_rsrc((const uint16_t*)p.q + (int64_t)b * p.q_sb + (int64_t)h * p.q_sh +
                                           (int64_t)(q0 + wrow0) * p.q_sr,
                                       (q_rows - 1) * q_rs + D * 2);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) qreg[kk] = buf_load16(qrs, lq * q_rs + (kk * 16 + hh * 8) * 2);
        } else {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                qreg[kk] = *(const uint4*)((const char*)smem + (q_lds - smem_addr) + k_lane + kk * 2 * 16 * 16);
        }
        if (p.neg) {
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) qreg[kk] = negate8(qreg[kk]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
        sh_run = kNegInf;
        l_run = 0.f;
        lr_run = 0.f;
        if (!ANYMASK && has_next) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): Q area reads done
            load_q(nP, ns);
        }
        scores(cur, sA);  // unconditional, so that no score register stays live across items
        if (!ANYMASK && first_item) {
            // K block 1 (K waves) and V block 0 (V waves) before the first step
            const int later = grp == 0 ? max(n_kv - 2, 0) : max(n_kv - 1, 0);
            pp_barrier_of<NDMA, NQDMA>(later * NDMA + (has_next ? NQDMA : 0));
        }
        first_item = false;
        if (ANYMASK && last_tile >= 0) {
            // the bias of block 0 (loaded after this wave's last bias read), then
            // the next block's load into the area just read
            __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0)
            MaskRead bv = bias_read(0);
#pragma unroll
            for (int i = 0; i < NBRD; ++i) {
                const MaskRead cv = bv;
                if (i + 1 < NBRD) bv = bias_read(i + 1);
                bias_add(sA, i, cv);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): bias reads done
            bias_next();
            kv_after_bias = false;
        }

        // End of step t: the wave's next block into the ring (a K block three
        // ahead of the compute goes where the K block read in the previous step
        // was, a V block two ahead where the V block of the previous step was;
        // both readers are behind the last barrier), then the wait for the
        // wave's older loads (the blocks the next step reads, and the next
        // item's Q^T) and the barrier.  In the first step of an item the K block
        // of the stage being refilled was also read in this step (the item's
        // first scores), so the barrier comes first there.
        // Float mask: a step that read a bias block (the next block is one this
        // wave computes) first issues the cursor's next bias block, before the
        // K/V load, so that section 2 of the next iteration waits for it with
        // the K/V load still in flight.
        auto step_end = [&](int t, bool bias_read_here) {
            const bool bl = ANYMASK && bias_read_here;
            if (t == 0) {
                pp_barrier<0>();
                const bool bi = bl && bias_next();
                const bool kv = load_next();
                if (bi) kv_after_bias = kv;
            } else {
                const bool bi = bl && bias_next();
                const bool kv = load_next();
                if (bi) {
                    kv_after_bias = kv;
                    if (kv)
                        pp_barrier<NDMA + NBDMA>();
                    else
                        pp_barrier<NBDMA>();
                } else if (kv) {
                    pp_barrier<NDMA>();
                } else {
                    pp_barrier<0>();
                }
            }
            cur = advance(cur);
        };
        // Blocks this wave takes part in, two per trip so the score buffers swap
        // roles without copies.  Reads and uses of the operand arrays are
        // unconditional here, so none stays live across the loop (after the
        // last block the next scores are computed from whatever the next stage
        // holds and unused).
        auto step = [&](int t, f32x16_t* sc, f32x16_t* sn) {
            const bool edge = (t * BN + BN > Sb) || (CAUSAL && t * BN + BN - 1 > q0 + wrow0 + coff);
            if (edge) mask_scores(t, sc);
            iteration(cur, advance(cur), sc, sn);
            step_end(t, t + 1 <= last_tile);
        };
        for (int t = 0; t <= last_tile; t += 2) {
            step(t, sA, sB);
            if (t + 1 > last_tile) break;
            step(t + 1, sB, sA);
        }
        // Blocks past this wave's rows: loads and barriers only.
        for (int t = last_tile + 1; t < nsteps; ++t) step_end(t, false);

        // Epilogue: O = O^T / l per lane (this lane's query), rounded to nearest-even,
        // with l the sum of the same rounded weights that multiplied V (a row dominated
        // by one weight then keeps that weight's rounding out of its output); lse takes
        // the sum of the fp32 weights.
        const float l_tot = pair32_sum(l_run);
        const float lr_tot = pair32_sum(lr_run);
        const float inv = (lr_tot == 0.f) ? 0.f : 1.f / lr_tot;
        const int o_rs = (int)(p.o_sr * 2);
        int lrow = wrow0 + lq;
        asm volatile("" : "+v"(lrow));  // per-lane store offsets computed here, not kept across the loop
        const auto ors = make_rsrc((uint16_t*)p.o + (VARQ ? 0 : (int64_t)b * p.o_sb) + (int64_t)h * p.o_sh +
                                       (tok0 + q0) * p.o_sr,
                                   (qrows - 1) * o_rs + D * 2);
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
            const auto lrs = make_rsrc(p.lse + (VARQ ? 0 : (int64_t)b * p.lse_sb) + (int64_t)h * p.lse_sh + tok0 + q0,
                                       qrows * 4);
            buf_store4(lse, lrs, lrow * 4);
        }
        P = nP;
        s = ns;
    }
}

// Compute units of the current device (cached per device).
inline int pp_device_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

template <typename Tr, int D, bool CAUSAL, int MASK = MASK_NONE, bool PAGED = false, bool VARQ = false>
hipError_t launch_prefill_pp(const AttnParams& p, hipStream_t stream) {
    PPWork w;
    w.nbh = p.Hq * p.B;
    w.nq = (p.L + kPPBlockM - 1) / kPPBlockM;
    w.n_pairs = w.nbh * ((w.nq + 1) / 2);
    if (w.n_pairs <= 0) return hipSuccess;
    const int grid = min(w.n_pairs, pp_device_cus());
    const int npp = (w.nq + 1) / 2;
    const auto pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
    const auto log2i = [](int v) { int l = 0; while ((1 << l) < v) ++l; return l; };
    // (with a mask the head-major numbering measured faster: 228 against 245 us
    // on the ALiBi workload, while without one the two take the same time and
    // this one re-reads less K/V: E=96 fetch 209 MB against 311 MB)
    w.xcd = (MASK == MASK_NONE && p.Hq % 8 == 0 && grid % 8 == 0 && pow2(npp) && pow2(p.B)) ? 1 : 0;
    w.npp_log2 = log2i(npp);
    w.b_log2 = log2i(p.B);
    hipLaunchKernelGGL((prefill_pp_kernel<Tr, D, CAUSAL, MASK, PAGED, VARQ>), dim3((unsigned)grid), dim3(512), 0, stream, p, w);
    return hipGetLastError();
}

}  // namespace sdpa

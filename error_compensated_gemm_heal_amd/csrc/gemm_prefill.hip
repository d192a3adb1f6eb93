// Prefill-shaped FP32-accurate GEMM on gfx950 16-bit MFMA.
//
// HEAL paper, section 3, "Mitigating GEMM Truncation via FP16 Promotion and
// Algebraic Compensation": each FP32 operand is written as an FP16 value
// plus an FP16 residual shifted by 2^10, and the product is expanded into
// 16-bit products with FP32 accumulation.  With both operands in FP32 the
// expansion keeps three products:
//     C = A_hi.B_hi + 2^-10 (A_hi.B_lo + A_lo.B_hi)
// (the lo.lo term is 2^-20 of the result and is dropped).
//
// Kernel structure (MFMA-bound; 3 x 2MNK flops on the 16-bit pipe):
//  * operands arrive packed by the split kernels: per row, each 32-wide k
//    block is one 128-byte line [32 hi | 32 res] fp16, zero-padded to whole
//    tiles, so the main loop has no bounds checks;
//  * FP16's narrow range (the same paragraph: handled by targeted
//    rescaling) is met by normalizing every operand row by a power of two:
//    its largest magnitude lies in [2^14, 2^15), and its residual is stored
//    at its own scale, res = fp16(x' - hi), which equals the paper's
//    lo 2^-10 for every element above 2^-17 of its row's largest.  So all
//    three products accumulate into one fp32 accumulator per output with no
//    scaling in the main loop, and the epilogue multiplies each output by
//    2^-(e_a[m] + e_b[n]) (exact, barring fp32 underflow): the result does
//    not depend on the operands' absolute scale;
//  * block tile 256 x 256 x 32, 4 waves in a 2 x 2 grid of 128 x 128 wave
//    tiles, each 4 x 4 tiles of v_mfma_f32_32x32x16_f16 (256 accumulator
//    registers per wave); a wave issues 96 MFMAs per k tile for 32 16-byte
//    LDS reads;
//  * k tiles move HBM -> LDS by buffer loads that write LDS directly (16
//    bytes per lane, no register staging) into two 64 KB stages;
//  * software pipeline with one barrier per k tile, placed mid-tile: the
//    MFMAs of k16 step 0 run while step 1's fragments are read; then the
//    barrier (tile t+1 landed, stage t free); then the MFMAs of step 1 run
//    while tile t+1's step-0 fragments are read and tile t+2's loads are
//    issued into the freed stage, so neither LDS latency nor the loads sit on
//    the MFMA critical path at tile boundaries;
//  * LDS rows are the packed 128-byte lines with their eight 16-byte chunks
//    XOR-swizzled by (row / 2) % 8, so the fragment reads of 16 consecutive
//    rows hit distinct banks with no padding;
//  * with a 16-bit weight (binary16 values, packed with zero lo planes) the
//    B_lo fragments are not read and the A_hi.B_lo product is skipped: the
//    paper's own two-product form, 2/3 of the MFMAs; the one-product mode
//    (plain FP16, no compensation) keeps A_hi.B_hi alone;
//  * when the grid would fill at most half the chip, the k range is split in
//    two and both halves add into a zeroed C with fp32 atomics; two addends
//    commute exactly, so the result does not depend on their order;
//  * block -> tile order keeps the blocks that share a B tile on one XCD
//    (blocks are dealt to the 8 XCDs round-robin), so B is read from HBM once
//    and re-served from that XCD's L2;
//  * the BF16 three-way mode (X3) splits both operands as x = b0 + b1 + b2
//    in BF16 (packed per 32-wide k block as [32 b0 | 32 b1 | 32 b2]) and
//    keeps the six products b_i.c_j with i + j <= 2 on the BF16 MFMA, one
//    fp32 accumulator.  It runs as a one-product GEMM over a virtual
//    reduction six times as long: virtual k tile 6 kb + j stages A's plane
//    (0,0,1,0,1,2)[j] and B's plane (0,1,0,2,1,0)[j] of block kb (64-byte
//    LDS rows on both sides); the repeated planes are re-read from L2;
//  * the Q/K/V projection epilogue (QKV) quantizes instead of storing: with
//    heads of 128 outputs, a wave's 128 columns are one head, so each
//    (token, head) row's maximum is a reduction over the wave's registers and
//    the 32 lanes of its half, and the INT16 codes and scale are written
//    straight to Q or to the K/V cache slot, with the standalone quantizer's
//    arithmetic (identical codes, and no fp32 product in memory);
//  * in the one-product mode an activation packed per call keeps its hi
//    parts alone (AH): 64-byte LDS rows for A, half its staging.
#include <utility>

#include "heal_internal.h"

namespace heal {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int WM = 128, WN = 128;           // wave tile
constexpr int TM = WM / 32, TN = WN / 32;   // 32x32 MFMA tiles per wave
constexpr int ROWB = 128;                   // LDS bytes per row: 32 hi + 32 lo fp16 (swizzled)
constexpr int NSTAGE = 2;
// Operand rows in LDS: 128 bytes (hi | lo), or 64 bytes for a single 16-bit
// plane (B in the hi-only form of a 16-bit weight; both operands in the BF16
// three-way mode), then 16 rows per 1 KB DMA block
constexpr int rowb(bool one_plane) { return one_plane ? 64 : ROWB; }
constexpr int stage_bytes(bool ahi, bool bhi) { return BM * rowb(ahi) + BN * rowb(bhi); }   // 64, 48 or 32 KB

// The INT16 epilogue's LDS: two wave tiles of 128 rows x 128 fp32 (row
// stride padded to 132 floats against bank conflicts), then 256 token slots.
constexpr int QKV_LD = 132;
constexpr int QKV_TILE_FLOATS = 128 * QKV_LD;
constexpr int QKV_SLOTS_OFF = 2 * QKV_TILE_FLOATS * 4;
constexpr int QKV_LDS = QKV_SLOTS_OFF + 256 * 8;   // 137 KB
constexpr int lds_base(bool ahi, bool bhi, bool qkv) {
    return qkv && QKV_LDS > NSTAGE * stage_bytes(ahi, bhi) ? QKV_LDS : NSTAGE * stage_bytes(ahi, bhi);
}
// After the stages (or the INT16 epilogue's tiles): the tile's 256 A and 256
// B row exponents (none in the BF16 mode)
constexpr int dyn_lds(bool ahi, bool bhi, bool qkv, bool x3) { return lds_base(ahi, bhi, qkv) + (x3 ? 0 : 2048); }

// HBM byte offset of virtual k tile kt in a three-way BF16 packed row: block
// kt / 6 (192 bytes), plane (planes >> 4 (kt % 6)) & 15 of it (64 bytes)
constexpr uint32_t X3_PLANES_A = 0x210100u;   // j = 0..5 -> 0, 0, 1, 0, 1, 2
constexpr uint32_t X3_PLANES_B = 0x012010u;   // j = 0..5 -> 0, 1, 0, 2, 1, 0
__device__ __forceinline__ uint32_t x3_koff(int kt, uint32_t planes) {
    const int kb = kt / 6, j = kt - 6 * kb;
    return (uint32_t)kb * 192u + ((planes >> (4 * j)) & 0xFu) * 64u;
}

// s_waitcnt immediate: at most n vector memory operations outstanding
// (vmcnt in bits 3:0 and 15:14); expcnt and lgkmcnt not waited on.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 32x32x16 MFMA on fp16 operands, or on the same registers read as bf16
template <bool BF16>
__device__ __forceinline__ void mfma32(const half8& a, const half8& b, floatx16& c) {
    if constexpr (BF16)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                    0, 0, 0);
    else
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// NP: products per k step.  3: A_hi.B_hi + A_hi.B_res + A_res.B_hi;
// 2: B is a 16-bit weight (no residual), A_hi.B + A_res.B;
// 1: plain FP16, A_hi.B_hi.  BHI / AH: B / A is staged as its hi parts alone
// (64-byte LDS rows): a 16-bit weight, and both operands in the one-product
// mode.  The packed source rows hold a_kstep / b_kstep bytes per 32-wide k
// block (128: hi and residual; 64: hi-only packing), so the one-product mode
// copies just the hi half of hi/residual rows.  X3: the BF16 three-way mode
// (NP = 1 over the virtual reduction, single planes).  QKV: the INT16
// epilogue for heads of 128 outputs (not with SPLIT).
template <bool SPLIT, int NP, bool BHI, bool X3, bool QKV, bool AH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_prefill_kernel(const unsigned char* __restrict__ Apk, const unsigned char* __restrict__ Bpk,
                         const int* __restrict__ ea, const int* __restrict__ eb,
                         float* __restrict__ C, int64_t ldc, int M, int N, int Kp,
                         int tiles_m, int tiles_n, uint32_t a_kstep, uint32_t b_kstep, QkvDst qkv) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    static_assert(!BHI || NP < 3, "a hi-only B has no lo planes");
    static_assert(!X3 || (NP == 1 && BHI), "the three-way mode is one product over single planes");
    static_assert(!(QKV && SPLIT), "the INT16 epilogue needs whole sums");
    static_assert(!AH || (NP == 1 && !X3), "a hi-only A goes with the one-product mode");
    constexpr bool AHI = X3 || AH;
    constexpr int STAGE = stage_bytes(AHI, BHI);
    constexpr int AROWB = rowb(AHI);
    constexpr int BROWB = rowb(BHI);
    constexpr int A_REGION = BM * AROWB;
    constexpr int A_DMA = BM * AROWB / 1024 / 4;   // 1 KB DMA blocks per wave per tile (A)
    constexpr int B_DMA = BN * BROWB / 1024 / 4;   // 1 KB DMA blocks per wave per tile (B)
    int* const exp_lds = reinterpret_cast<int*>(smem + lds_base(AHI, BHI, QKV));

    // ---- XCD-aware tile order (tm fastest, then tn, then the k half) -------
    const int nblk = tiles_m * tiles_n * (SPLIT ? 2 : 1);
    int bid = blockIdx.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
    const int tm = bid % tiles_m;
    const int tn = (bid / tiles_m) % tiles_n;
    const int half_k = SPLIT ? bid / (tiles_m * tiles_n) : 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the tile's row exponents, loaded first and parked in LDS for the epilogue
    int ea_v = 0, eb_v = 0;
    if constexpr (!X3) {
        ea_v = ea[tm * BM + tid];
        eb_v = eb[tn * BN + tid];
    }
    // wave index as a scalar: DMA destinations and offsets must be wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    // HBM row bytes: Kp hi + Kp lo fp16; Kp fp16 (hi-only); 3 Kp bf16 (X3)
    // packed row strides: 3 Kp bf16 (X3, no pad), or the padded hi-only / hi-res rows
    const uint32_t rowbytes = X3 ? (uint32_t)Kp * 6u : (uint32_t)(Kp / 32) * a_kstep + (uint32_t)kPackRowPad;
    const uint32_t browbytes = X3 ? (uint32_t)Kp * 6u : (uint32_t)(Kp / 32) * b_kstep + (uint32_t)kPackRowPad;
    const int nkt_all = (X3 ? 6 : 1) * (Kp / BK);
    const int kt_begin = SPLIT ? half_k * (nkt_all / 2) : 0;
    const int kt_end = SPLIT ? (half_k ? nkt_all : nkt_all / 2) : nkt_all;
    const int nkt = kt_end - kt_begin;

    // ---- DMA: wave w fills the 1 KB blocks b = w + 4 i (8 rows each) ------
    // Lane L writes LDS row L/8, slot L%8 of its block; the slot holds chunk
    // (L%8) ^ sw(row) with sw(row) = (row / 2) % 8.  b has the parity of w, so
    // sw depends on the lane and the wave only.
    const int drow = lane >> 3;
    const int dsw = ((wave & 1) << 2) | (drow >> 1);
    const uint32_t dma_slot = (uint32_t)((lane & 7) ^ dsw) * 16u;
    // hi-only B: lane L writes row L/4, slot L%4 of a 16-row block, holding
    // chunk (L%4) ^ ((row / 4) % 4); 16 rows per block keep that lane-only
    const int drow_1 = lane >> 2;
    const uint32_t slot_1 = (uint32_t)((lane & 3) ^ ((drow_1 >> 2) & 3)) * 16u;
    const uint32_t dma_voff_b = BHI ? (uint32_t)drow_1 * browbytes + slot_1 : (uint32_t)drow * browbytes + dma_slot;
    const uint32_t dma_voff_a = AHI ? (uint32_t)drow_1 * rowbytes + slot_1 : (uint32_t)drow * rowbytes + dma_slot;
    constexpr int A_ROWS_PER_DMA = 1024 / AROWB;
    constexpr int B_ROWS_PER_DMA = 1024 / BROWB;
    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(Apk + (int64_t)tm * BM * rowbytes, BM * rowbytes);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(Bpk + (int64_t)tn * BN * browbytes, BN * browbytes);

#define HEAL_DMA_TILE(kt_, stage_)                                                                    \
    do {                                                                                              \
        unsigned char* st_ = smem + (stage_) * STAGE;                                                 \
        const uint32_t koff_a_ = X3 ? x3_koff(kt_, X3_PLANES_A) : (uint32_t)(kt_) * a_kstep;          \
        const uint32_t koff_b_ = X3 ? x3_koff(kt_, X3_PLANES_B) : (uint32_t)(kt_) * b_kstep;          \
        _Pragma("unroll") for (int i = 0; i < A_DMA; ++i) {                                           \
            const int b_ = wave + 4 * i;                                                              \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_ptr)(st_ + b_ * 1024), 16, dma_voff_a, \
                                                     (uint32_t)(A_ROWS_PER_DMA * b_) * rowbytes + koff_a_, \
                                                     0, 0);                                           \
        }                                                                                             \
        _Pragma("unroll") for (int i = 0; i < B_DMA; ++i) {                                           \
            const int b_ = wave + 4 * i;                                                              \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, (lds_ptr)(st_ + A_REGION + b_ * 1024), 16, \
                                                     dma_voff_b,                                      \
                                                     (uint32_t)(B_ROWS_PER_DMA * b_) * browbytes + koff_b_, \
                                                     0, 0);                                           \
        }                                                                                             \
    } while (0)

    // ---- fragment reads: lane reads row (l % 32) of a 32-row tile, chunk
    //      2 ks + l / 32 (hi) or 4 + 2 ks + l / 32 (lo), at its swizzled slot
    const int sw = (lane >> 1) & 7;
    const int a_row = (wm * WM + (lane & 31)) * AROWB;
    const int b_row = A_REGION + (wn * WN + (lane & 31)) * BROWB;
    int slot_off[2][2];   // [ks][hi/lo]
    int slot_off_a[2];    // A hi chunk: the 128-byte-row slots, or the single-plane swizzle (row / 4) % 4
    int slot_off_b[2];    // B hi chunk, likewise
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int p = 0; p < 2; ++p) slot_off[ks][p] = ((4 * p + 2 * ks + (lane >> 5)) ^ sw) * 16;
        const int one_plane = ((2 * ks + (lane >> 5)) ^ (((lane & 31) >> 2) & 3)) * 16;
        slot_off_a[ks] = AHI ? one_plane : slot_off[ks][0];
        slot_off_b[ks] = BHI ? one_plane : slot_off[ks][0];
    }

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // fragments of one k16 step: ah/al (A hi, A lo), bh/bl (B hi, B lo)
#define HEAL_FRAGS(ah_, al_, bh_, bl_, ks_)                                                              \
    do {                                                                                                 \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                                 \
            ah_[i] = *reinterpret_cast<const half8*>(base + a_row + i * 32 * AROWB + slot_off_a[ks_]);  \
            if constexpr (NP >= 2)                                                                       \
                al_[i] = *reinterpret_cast<const half8*>(base + a_row + i * 32 * ROWB + slot_off[ks_][1]); \
        }                                                                                                \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                                 \
            bh_[j] = *reinterpret_cast<const half8*>(base + b_row + j * 32 * BROWB + slot_off_b[ks_]);   \
            if constexpr (NP == 3)                                                                       \
                bl_[j] = *reinterpret_cast<const half8*>(base + b_row + j * 32 * ROWB + slot_off[ks_][1]); \
        }                                                                                                \
    } while (0)
    // The k16 step's work is issued in 16 slots separated by scheduling
    // barriers (the scheduler does not keep an interleave of MFMAs, copies and
    // LDS reads by itself once nothing but loads feeds the MFMAs): slot q runs
    // NP MFMAs of the product-major sequence m = 16 p + 4 i + j (each product
    // sweeps the 16 output tiles, so an accumulator is re-read 16 MFMAs later)
    // and its share of the next fragment reads (and, in the second half of a
    // tile, of the next tile's copies).
    constexpr int NM_ = 16 * NP;
    constexpr int NR_ = TM + (NP >= 2 ? TM : 0) + TN + (NP == 3 ? TN : 0);
#define HEAL_SLOT_MFMAS(q_, ah_, al_, bh_, bl_)                                                           \
    _Pragma("unroll") for (int m = (q_) * NM_ / 16; m < ((q_) + 1) * NM_ / 16; ++m) {                    \
        const int p = m >> 4, i = (m >> 2) & 3, j = m & 3;                                               \
        if (p == 0) mfma32<X3>(ah_[i], bh_[j], acc[i][j]);                                              \
        else if (NP == 3 && p == 1) mfma32<false>(ah_[i], bl_[j], acc[i][j]);                           \
        else mfma32<false>(al_[i], bh_[j], acc[i][j]);                                                  \
    }
#define HEAL_SLOT_READS(q_, base_, ks_, ah_, al_, bh_, bl_)                                               \
    _Pragma("unroll") for (int r0 = (q_) * NR_ / 16; r0 < ((q_) + 1) * NR_ / 16; ++r0) {                 \
        int r = r0;                                                                                      \
        if (r < TM) { ah_[r] = *reinterpret_cast<const half8*>(base_ + a_row + r * 32 * AROWB + slot_off_a[ks_]); continue; } \
        r -= TM;                                                                                         \
        if constexpr (NP >= 2) {                                                                         \
            if (r < TM) { al_[r] = *reinterpret_cast<const half8*>(base_ + a_row + r * 32 * ROWB + slot_off[ks_][1]); continue; } \
            r -= TM;                                                                                     \
        }                                                                                                \
        if (r < TN) { bh_[r] = *reinterpret_cast<const half8*>(base_ + b_row + r * 32 * BROWB + slot_off_b[ks_]); continue; } \
        r -= TN;                                                                                         \
        if constexpr (NP == 3) bl_[r] = *reinterpret_cast<const half8*>(base_ + b_row + r * 32 * ROWB + slot_off[ks_][1]); \
    }
    // Pipeline, one barrier per k tile placed mid-tile:
    //   phase 1 of tile t: MFMAs of k16 step 0 while step 1's fragments load;
    //   sync: this wave's reads of stage t done, tile t+1's DMA landed, barrier;
    //   phase 2: MFMAs of step 1 while tile t+1's step-0 fragments load and
    //   tile t+2's DMA refills the stage tile t used.
    half8 ah0[TM], al0[TM], bh0[TN], bl0[TN], ah1[TM], al1[TM], bh1[TN], bl1[TN];
    HEAL_DMA_TILE(kt_begin, 0);
    if (nkt > 1) {
        HEAL_DMA_TILE(kt_begin + 1, 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(A_DMA + B_DMA));   // tile 0 landed, tile 1 in flight
    } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
    }
    if constexpr (!X3) {
        exp_lds[tid] = ea_v;
        exp_lds[256 + tid] = eb_v;
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    {
        const unsigned char* base = smem;
        HEAL_FRAGS(ah0, al0, bh0, bl0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int t = 0; t < nkt; ++t) {
        {   // phase 1
            const unsigned char* base = smem + (t & 1) * STAGE;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                HEAL_SLOT_MFMAS(q, ah0, al0, bh0, bl0)
                HEAL_SLOT_READS(q, base, 1, ah1, al1, bh1, bl1)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (t + 1 < nkt) {   // sync (uniform across the block)
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        {   // phase 2 (branch-free so the loads interleave with the MFMAs): near
            // the end the tile indices clamp to the last tile, whose re-fetch
            // writes bytes identical to the ones already in LDS.  Slots: MFMAs,
            // copies, next fragment reads
            const int kt2 = kt_begin + min(t + 2, nkt - 1);
            unsigned char* const st2 = smem + (t & 1) * STAGE;
            const uint32_t koff_a2 = X3 ? x3_koff(kt2, X3_PLANES_A) : (uint32_t)kt2 * a_kstep;
            const uint32_t koff_b2 = X3 ? x3_koff(kt2, X3_PLANES_B) : (uint32_t)kt2 * b_kstep;
            const unsigned char* base = smem + (min(t + 1, nkt - 1) & 1) * STAGE;
            constexpr int ND = A_DMA + B_DMA;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                HEAL_SLOT_MFMAS(q, ah1, al1, bh1, bl1)
#pragma unroll
                for (int d = q * ND / 16; d < (q + 1) * ND / 16; ++d) {
                    if (d < A_DMA) {
                        const int b_ = wave + 4 * d;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_ptr)(st2 + b_ * 1024), 16, dma_voff_a,
                                                                 (uint32_t)(A_ROWS_PER_DMA * b_) * rowbytes + koff_a2, 0, 0);
                    } else {
                        const int b_ = wave + 4 * (d - A_DMA);
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, (lds_ptr)(st2 + A_REGION + b_ * 1024), 16,
                                                                 dma_voff_b,
                                                                 (uint32_t)(B_ROWS_PER_DMA * b_) * browbytes + koff_b2,
                                                                 0, 0);
                    }
                }
                HEAL_SLOT_READS(q, base, 0, ah0, al0, bh0, bl0)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // no LDS write of this block may land after it ends
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#undef HEAL_FRAGS
#undef HEAL_SLOT_MFMAS
#undef HEAL_SLOT_READS
#undef HEAL_DMA_TILE

    // ---- epilogue: store (or atomic add of one k half) ----------------------
    // undo the row normalization: output (row, col) times 2^-(ea[row] + eb[col]),
    // exact barring fp32 underflow; the exponents come from LDS.  (The INT16
    // epilogue scales each value as it stages it.)
    const int ln = __lane_id();   // recomputed (mbcnt): no lane value is held over the main loop
    if constexpr (!X3 && !QKV) {
        __syncthreads();   // the exponents' LDS writes are visible (also when the loop had one tile)
        const int rl = wm * WM + (ln >> 5) * 4, cl = wn * WN + (ln & 31);
        int ebc[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) ebc[j] = exp_lds[256 + cl + j * 32];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            int4 er[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) er[q] = *reinterpret_cast<const int4*>(exp_lds + rl + i * 32 + q * 8);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[i][j][4 * q + 0] = __builtin_ldexpf(acc[i][j][4 * q + 0], -(er[q].x + ebc[j]));
                    acc[i][j][4 * q + 1] = __builtin_ldexpf(acc[i][j][4 * q + 1], -(er[q].y + ebc[j]));
                    acc[i][j][4 * q + 2] = __builtin_ldexpf(acc[i][j][4 * q + 2], -(er[q].z + ebc[j]));
                    acc[i][j][4 * q + 3] = __builtin_ldexpf(acc[i][j][4 * q + 3], -(er[q].w + ebc[j]));
                }
        }
    }
    if constexpr (QKV) {
        // The output goes through LDS (the operand stages are free now): in
        // pass p the two waves of wave column p write their 128 x 128 fp32
        // tiles (one head each: heads are 128 outputs), then all four waves
        // quantize those 256 (token, head) rows, one row per half wave (32
        // lanes x 4 values), with the standalone quantizer's arithmetic.  The
        // block's token slots are staged once.
        __syncthreads();   // also makes the exponents' LDS writes visible
        const int rl = wm * WM + (ln >> 5) * 4, cl = wn * WN + (ln & 31);
        int ebc[TN] = {};
        if constexpr (!X3) {
#pragma unroll
            for (int j = 0; j < TN; ++j) ebc[j] = exp_lds[256 + cl + j * 32];
        }
        float* tile = reinterpret_cast<float*>(smem);
        int64_t* slot_lds = reinterpret_cast<int64_t*>(smem + QKV_SLOTS_OFF);
        {
            const int r = tm * BM + tid;
            slot_lds[tid] = r < M ? qkv.slots[r] : -1;
        }
        bool bad_slot = false;
#pragma unroll 1
        for (int p = 0; p < 2; ++p) {
            const int colp = tn * BN + p * WN;   // head colp / 128; block-uniform
            if (colp >= N) break;                // N is a multiple of 128
            if (wn == p) {
                float* t = tile + wm * QKV_TILE_FLOATS;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    int er[16] = {};
                    if constexpr (!X3) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int4 v = *reinterpret_cast<const int4*>(exp_lds + rl + i * 32 + q * 8);
                            er[4 * q + 0] = v.x;
                            er[4 * q + 1] = v.y;
                            er[4 * q + 2] = v.z;
                            er[4 * q + 3] = v.w;
                        }
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int rr = (ln >> 5) * 4 + i * 32 + (e >> 2) * 8 + (e & 3);
                            t[rr * QKV_LD + j * 32 + (ln & 31)] =
                                X3 ? acc[i][j][e] : __builtin_ldexpf(acc[i][j][e], -(er[e] + ebc[j]));
                        }
                }
            }
            __syncthreads();
            const int hd = colp / 128;
            const bool is_q = hd < qkv.hq;
            const bool is_k = !is_q && hd < qkv.hq + qkv.hkv;
            const int hk = is_q ? hd : (is_k ? hd - qkv.hq : hd - qkv.hq - qkv.hkv);
            int16_t* const cbase = is_q ? qkv.qc : (is_k ? qkv.kc : qkv.vc);
            float* const sbase = is_q ? qkv.qs : (is_k ? qkv.ks : qkv.vs);
            const int hcount = is_q ? qkv.hq : qkv.hkv;
            const int c4 = 4 * (ln & 31);
#pragma unroll 8
            for (int it = 0; it < 32; ++it) {
                const int r = wave * 64 + it * 2 + (ln >> 5);   // 0..255: tile r / 128, row r % 128
                const int rl = r;                                 // row in the block (tile 0: wm 0, tile 1: wm 1)
                const float4 x = *reinterpret_cast<const float4*>(tile + (r >> 7) * QKV_TILE_FLOATS +
                                                                  (r & 127) * QKV_LD + c4);
                float m = fmaxf(fmaxf(__builtin_fabsf(x.x), __builtin_fabsf(x.y)),
                                fmaxf(__builtin_fabsf(x.z), __builtin_fabsf(x.w)));
                m = max_half(m);
                if (tm * BM + rl >= M) continue;
                int64_t dst_row = tm * BM + rl;   // Q: the token row
                if (!is_q) {
                    dst_row = slot_lds[rl];
                    if (dst_row < 0) continue;                                   // a padding token
                    if (dst_row >= qkv.num_slots) { bad_slot = true; continue; }
                }
                const int64_t idx = dst_row * hcount + hk;
                if ((ln & 31) == 0) sbase[idx] = (m == 0.0f) ? 0.0f : __fdiv_rn(m, 32767.0f);
                // a zero row (m = 0, all x = 0) divides by 1 and gives zero codes
                const float dm = (m == 0.0f) ? 1.0f : m;
                short4 q;
                q.x = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x.x), dm));
                q.y = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x.y), dm));
                q.z = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x.z), dm));
                q.w = (short)__builtin_rintf(__fdiv_rn(__fmul_rn(32767.0f, x.w), dm));
                *reinterpret_cast<short4*>(cbase + idx * 128 + c4) = q;
            }
            __syncthreads();   // the tiles are read before the next pass overwrites them
        }
        if (bad_slot && qkv.status) atomicOr(qkv.status, (uint32_t)HEAL_FLAG_SLOT_RANGE);
        return;
    }
    if (!SPLIT && (tm + 1) * BM <= M && (tn + 1) * BN <= N && ldc < ((int64_t)1 << 26)) {
        // a whole tile (block-uniform): no bounds checks.  Each store is a
        // wave-uniform row address (the wave tile's corner plus r ldc, scalar
        // arithmetic), the lane's 32-bit byte offset (its row in the group of
        // four, its column) and the 32-column tile as an immediate offset.
        // (The k halves' atomic adds keep the form below: issued back to
        // back in this form they measured 1-2% slower per call.)
        char* const wbase = reinterpret_cast<char*>(C + (int64_t)(tm * BM + wm * WM) * ldc + (tn * BN + wn * WN));
        const uint32_t loff = (uint32_t)(((ln >> 5) * 4 * (int)ldc + (ln & 31)) * 4);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                char* const rb = wbase + (int64_t)(i * 32 + (e >> 2) * 8 + (e & 3)) * ldc * 4;
#pragma unroll
                for (int j = 0; j < TN; ++j) *reinterpret_cast<float*>(rb + loff + j * 128) = acc[i][j][e];
            }
        return;
    }
    // a partial tile: every element checked
    const int row0 = tm * BM + wm * WM + (ln >> 5) * 4;
    const int col0 = tn * BN + wn * WN + (ln & 31);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = col0 + j * 32;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = row0 + i * 32 + (e >> 2) * 8 + (e & 3);
                if (row < M) {
                    float* dst = C + (int64_t)row * ldc + col;
                    if (SPLIT)
                        unsafeAtomicAdd(dst, acc[i][j][e]);
                    else
                        *dst = acc[i][j][e];
                }
            }
        }
}

// C := 0 before the k halves add into it: rows by blockIdx.y (grid-stride),
// 16-byte stores where C's rows are 16-byte aligned
__global__ void zero_c_kernel(float* C, int64_t ldc, int64_t M, int64_t N) {
    const bool vec = ((reinterpret_cast<uintptr_t>(C) | (uintptr_t)(ldc * 4)) & 15) == 0;
    const int64_t n4 = vec ? N / 4 : 0;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float* row = C + m * ldc;
        for (int64_t i = t0; i < n4; i += step) reinterpret_cast<float4*>(row)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int64_t i = 4 * n4 + t0; i < N; i += step) row[i] = 0.0f;
    }
}

}  // namespace

bool prefill_ksplit(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    return tiles <= 128 && pack_kp(K) / BK >= 8;
}

hipError_t launch_gemm_prefill(const void* Apk, const void* Bpk, int nprod, bool b_hi, float* C, int64_t ldc,
                               int64_t M, int64_t N, int64_t K, hipStream_t s, const QkvDst* qkv, bool a_hi) {
    // two products go with a 16-bit (hi-only) B, three with a hi/lo B; 6 is
    // the BF16 three-way mode (both operands in its packed form)
    const bool x3 = nprod == 6;
    if (!x3 && (nprod < 1 || nprod > 3 || (nprod == 3 && b_hi) || (nprod == 2 && !b_hi))) return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t Kp = pack_kp(K);
    if (Kp == 0) return hipErrorInvalidValue;  // K == 0 is handled by the caller
    // one operand block must be addressable by a 32-bit buffer offset
    if ((int64_t)BM * (x3 ? Kp * 6 : pack_row_bytes(K)) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    // split the k range in two when the tiles fill at most half of the 256 CUs
    const bool split = prefill_ksplit(M, N, K);
    // the INT16 epilogue: heads of 128, whole sums, the 3- or 2-product form
    if (qkv && (split || x3 || nprod == 1 || qkv->d != 128 || N % 128 != 0)) return hipErrorInvalidValue;
    if (a_hi && (nprod != 1 || qkv)) return hipErrorInvalidValue;   // a hi-only A: the one-product mode
    // once per device (the attribute is per device); idempotent, so racing
    // first calls set the same value
    constexpr int kMaxDevices = 64;
    static bool attr_set[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!attr_set[dev]) {
        const std::pair<const void*, int> fns[10] = {
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<false, 3, false, false, false, false>), dyn_lds(false, false, false, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<true, 3, false, false, false, false>), dyn_lds(false, false, false, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<false, 2, true, false, false, false>), dyn_lds(false, true, false, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<true, 2, true, false, false, false>), dyn_lds(false, true, false, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<false, 1, true, true, false, false>), dyn_lds(true, true, false, true)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<true, 1, true, true, false, false>), dyn_lds(true, true, false, true)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<false, 3, false, false, true, false>), dyn_lds(false, false, true, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<false, 2, true, false, true, false>), dyn_lds(false, true, true, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<false, 1, true, false, false, true>), dyn_lds(true, true, false, false)},
            {reinterpret_cast<const void*>(&gemm_prefill_kernel<true, 1, true, false, false, true>), dyn_lds(true, true, false, false)}};
        for (const auto& f : fns) {
            const int bytes = f.second;
            hipError_t e = hipFuncSetAttribute(f.first, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
            if (e != hipSuccess) return e;
        }
        attr_set[dev] = true;
    }
    const unsigned char* a = static_cast<const unsigned char*>(Apk);
    const unsigned char* b = static_cast<const unsigned char*>(Bpk);
    // the row exponents follow each packed operand's rows (none in the BF16 mode)
    const int* ea = x3 ? nullptr
                       : reinterpret_cast<const int*>(a + (a_hi ? pack_data_bytes_hi(M, K) : pack_data_bytes(M, K)));
    const int* eb = x3 ? nullptr
                       : reinterpret_cast<const int*>(b + (b_hi ? pack_data_bytes_hi(N, K) : pack_data_bytes(N, K)));
    if (split) {
        const dim3 zg((unsigned)std::min<int64_t>((N + 1023) / 1024, 64), (unsigned)std::min<int64_t>(M, 1024));
        hipLaunchKernelGGL(zero_c_kernel, zg, dim3(256), 0, s, C, ldc, M, N);
    }
    const dim3 grid((unsigned)(tiles_m * tiles_n * (split ? 2 : 1)));
    const QkvDst none{};
    // bytes per 32-wide k block in the packed source rows
    const uint32_t a_kstep = a_hi ? 64u : 128u, b_kstep = b_hi ? 64u : 128u;
#define HEAL_PREFILL(SPLIT_, NP_, BHI_, X3_)                                                          \
    hipLaunchKernelGGL((gemm_prefill_kernel<SPLIT_, NP_, BHI_, X3_, false, false>), grid, dim3(256),  \
                       dyn_lds(X3_, BHI_, false, X3_), s, a, b, ea, eb, C, ldc, (int)M, (int)N, (int)Kp, tiles_m, tiles_n, \
                       a_kstep, b_kstep, none)
#define HEAL_PREFILL_1P(SPLIT_)                                                                       \
    hipLaunchKernelGGL((gemm_prefill_kernel<SPLIT_, 1, true, false, false, true>), grid, dim3(256),    \
                       dyn_lds(true, true, false, false), s, a, b, ea, eb, C, ldc, (int)M, (int)N, (int)Kp, tiles_m, tiles_n, \
                       a_kstep, b_kstep, none)
    if (qkv) {
        if (nprod == 3)
            hipLaunchKernelGGL((gemm_prefill_kernel<false, 3, false, false, true, false>), grid, dim3(256),
                               dyn_lds(false, false, true, false), s, a, b, ea, eb, C, ldc, (int)M, (int)N, (int)Kp, tiles_m,
                               tiles_n, a_kstep, b_kstep, *qkv);
        else
            hipLaunchKernelGGL((gemm_prefill_kernel<false, 2, true, false, true, false>), grid, dim3(256),
                               dyn_lds(false, true, true, false), s, a, b, ea, eb, C, ldc, (int)M, (int)N, (int)Kp, tiles_m,
                               tiles_n, a_kstep, b_kstep, *qkv);
        return hipGetLastError();
    }
    // the one-product mode stages the hi parts alone, from either packing
#define HEAL_PREFILL_NP(SPLIT_)                                                                       \
    do {                                                                                              \
        if (x3) HEAL_PREFILL(SPLIT_, 1, true, true);                                                  \
        else if (nprod == 3) HEAL_PREFILL(SPLIT_, 3, false, false);                                   \
        else if (nprod == 2) HEAL_PREFILL(SPLIT_, 2, true, false);                                    \
        else HEAL_PREFILL_1P(SPLIT_);                                                                 \
    } while (0)
    if (split) HEAL_PREFILL_NP(true);
    else HEAL_PREFILL_NP(false);
#undef HEAL_PREFILL_NP
#undef HEAL_PREFILL_1P
#undef HEAL_PREFILL
    return hipGetLastError();
}

}  // namespace heal

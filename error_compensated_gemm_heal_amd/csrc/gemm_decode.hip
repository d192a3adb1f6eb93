// Decode-shaped FP32-accurate GEMM (M <= 64) on gfx950 16-bit MFMA.
//
// Same arithmetic as the prefill kernel (HEAL paper, section 3, "Mitigating
// GEMM Truncation via FP16 Promotion and Algebraic Compensation"):
//     C = A_hi.B_hi + 2^-10 (A_hi.B_lo + A_lo.B_hi),  fp32 accumulation,
// but shaped for a skinny activation, where the weight is the traffic:
//  * W is read once from HBM as fp32 [N, K] (4 bytes per element, the same
//    bytes as its two fp16 parts) and split into hi/lo in registers, or as a
//    weight packed once by heal_pack_w (row-normalized hi and residual
//    parts, rows padded off power-of-two strides), which needs no split;
//  * FP16's narrow range (the same paragraph: handled by targeted
//    rescaling): every 128-wide k block of every activation row is
//    multiplied by the power of two 2^e that puts its largest magnitude in
//    [2^14, 2^15) before its split; the block's products accumulate in fresh
//    fp32 accumulators, which are folded into the running sums as
//    (acc_hh + 2^-10 acc_c) 2^-e once per block.  The result thus does not
//    depend on the activation's absolute scale (W is split as it is), and no
//    pass over the activation is needed before the split;
//  * the activation (<= 64 rows) is staged in 128-wide k blocks in a
//    double-buffered LDS tile, in MFMA operand order, so every operand read
//    is one conflict-free 16-byte LDS access; the block's 16 MT exponents
//    travel with it.  Up to 16 rows, each workgroup loads the next block into
//    registers while the current one is in use (each wave takes groups of
//    four rows, so a row's block maximum is a reduction inside one wave) and
//    normalizes and splits it itself: one launch in all.  Above 16 rows the
//    same holds where that work stays light; otherwise, where it would be
//    repeated by every workgroup, a first small kernel (decode_prep_kernel,
//    one workgroup per row) writes the blocks the same way into
//    operand-ordered planes once, and workgroups copy them into LDS with
//    direct-to-LDS loads;
//  * v_mfma_f32_16x16x32_f16 with the activation as the 16-row operand and W
//    as the 16-column operand (16 W rows per wave), so output columns are
//    consecutive lanes;
//  * inside each 32-wide k step, lane group g (lanes 16g..16g+15) carries
//    k = 8g..8g+7 (k = 4g..4g+3 and 16+4g..16+4g+3 where W is loaded element
//    by element): any k order is valid as long as both operands use it, and
//    this one keeps each lane's W values contiguous (one 16-byte load of
//    binary16 W or of each packed part, two of fp32).  The MFMA's sum over
//    its 32 k positions is not invariant under permuting them, so every
//    vector-loaded W (fp32, binary16, packed) uses the same order: a binary16
//    weight gives the bits of its fp32 copy;
//  * W for the next 8 k steps is always in flight: every step issues a
//    fixed number of W loads (the last steps re-read a clamped step), so the
//    number of loads outstanding at each block boundary is a constant;
//  * with fewer than 8 k chunks, each 128-row group of W visits its chunk's
//    k blocks in a rotated order, so that rows with a power-of-two stride do
//    not all hit the same HBM channels at once;
//  * split-K: the k range is cut into chunks chosen from (N, K) only.  Each
//    workgroup writes its chunk's partial outputs with write-through stores,
//    waits for them to complete, sets its (row block, chunk) flag to the
//    call's epoch the same way, and reads its row block's flags; a workgroup
//    that finds them all set sums the chunk partials in chunk order (its own
//    from registers, the others with loads that bypass the non-coherent L2)
//    and writes C.  Flags from earlier calls hold other epochs, so the
//    workspace needs no zeroing pass; no atomic read-modify-write, no second
//    launch, no L2 write-back, and the summation order of an output does not
//    depend on M or on arrival order: a decode-sized product does not change
//    with the batch it is computed in.
#include <type_traits>

#include "heal_internal.h"

namespace heal {

namespace {

constexpr int KA = 128;             // k block of activations per LDS buffer
constexpr int STEPS = KA / 32;      // k32 steps per block
constexpr int PF = 8;               // W prefetch distance in k32 steps (multiple of STEPS, <= 4 STEPS)
constexpr int NW = 4;               // waves per workgroup (8 with four row tiles: see nw_for)
constexpr int TARGET_WG = 512;      // workgroups aimed for (two per compute unit)
constexpr int ROWS_PER_WAVE = 16;
constexpr int DEC_ROWS = NW * ROWS_PER_WAVE;  // W rows per 4-wave group: the unit of the split-K plan
// Waves per workgroup (NWK): with the copied activation (M > 16) its block in
// LDS is as large as the weight block of 4 waves (four row tiles) or half of
// it (two), so 8 waves share it (half the activation bytes per weight byte)
// when the grid keeps enough workgroups: measured, four tiles gain at 224 and
// lose at 128; two tiles gain at 256 and lose at 224.  The split-K plan and
// each output's summation order do not depend on it.
constexpr int WIDE_MIN_WG4 = 192;
constexpr int WIDE_MIN_WG2 = 256;


// s_waitcnt immediate that waits until at most n vector memory operations
// are outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate that waits for all LDS operations (lgkmcnt 0) only.
constexpr int lgkmcnt0_imm() { return 0xF | (0x3 << 14) | (0x7 << 4); }

__device__ __forceinline__ void mfma16(const half8& a, const half8& b, floatx4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Bytes of one activation block: hi and lo planes of STEPS x MT x 64 lanes x 16 B.
template <int MT>
constexpr int block_bytes() { return 2 * STEPS * MT * 64 * 16; }

// Bytes of one activation block image: the two planes, then the exponents
// of its 16 MT rows (int32, padded to 256 bytes).
template <int MT>
constexpr int img_bytes() { return block_bytes<MT>() + 256; }

// ---- the first kernel (MT > 1): operand-ordered blocks with their exponents
// Workgroup (m, y) takes 16 blocks of row m of A (k in [2048 y, 2048 y +
// 2048)), one float4 of 4 consecutive k per lane: the 32 lanes of a half
// wave hold one 128-wide block, so the block's largest magnitude (after the
// optional 2^-kshift[k]) is a reduction inside the half wave.  It gives the
// block's exponent e; the lane writes its 4 values, x 2^(e - kshift[k]), split
// as hi = fp16, lo = fp16((x - hi) 2^10), into block b's image: plane p
// (0 = hi, 1 = lo), step s, tile t, lane 16 g + r holds, as 8 fp16, row
// 16 t + r at k = 128 b + 32 s + {4g .. 4g+3, 16+4g .. 16+4g+3} (K8, for a
// vector-loaded W: k = 128 b + 32 s + 8g .. 8g+7); then e at byte block_bytes + 4 m.  Rows >= M and k >= K are zero (exponent 0).  One
// load per thread: the kernel costs about one memory latency.
constexpr int PREP_T = 512;
template <int MT, bool AVEC, bool K8>
__global__ __launch_bounds__(PREP_T) void decode_prep_kernel(const float* __restrict__ A, int64_t lda, int M, int K,
                                                             int nblk, const int8_t* __restrict__ kshift,
                                                             unsigned char* __restrict__ out) {
    constexpr int BB = block_bytes<MT>();
    const int m = blockIdx.x;
    const int q = blockIdx.y * PREP_T + threadIdx.x;   // float4 slot: k = 4 q .. 4 q + 3
    const int t = m >> 4, r = m & 15;
    const float* a = A + (int64_t)m * lda;
    auto val = [&](int k) {
        return (m < M && k < K) ? __builtin_ldexpf(a[k], kshift ? -(int)kshift[k] : 0) : 0.0f;
    };
    const int k = 4 * q;
    float4 v;
    if (AVEC && m < M && k + 3 < K) {
        v = *reinterpret_cast<const float4*>(a + k);
        if (kshift) {
            v.x = __builtin_ldexpf(v.x, -(int)kshift[k]);
            v.y = __builtin_ldexpf(v.y, -(int)kshift[k + 1]);
            v.z = __builtin_ldexpf(v.z, -(int)kshift[k + 2]);
            v.w = __builtin_ldexpf(v.w, -(int)kshift[k + 3]);
        }
    } else {
        v = make_float4(val(k), val(k + 1), val(k + 2), val(k + 3));
    }
    float mx = fmaxf(fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)), fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
    mx = max_half(mx);
    if (q >= nblk * 32) return;   // past the last block (whole half waves)
    const int e = row_norm_exp(mx);
    // j = 8 s + 4 h + g: k = 128 b + 32 s + 16 h + 4 g; K8:
    // j = 8 s + 2 g + h: k = 128 b + 32 s + 8 g + 4 h
    const int b = q >> 5, j = q & 31;
    const int st = j >> 3, h = K8 ? (j & 1) : ((j >> 2) & 1), g = K8 ? ((j >> 1) & 3) : (j & 3);
    const float x[4] = {v.x, v.y, v.z, v.w};
    half4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        _Float16 hh, ll;
        split_one(__builtin_ldexpf(x[i], e), hh, ll);
        hi[i] = hh;
        lo[i] = ll;
    }
    unsigned char* blk = out + (int64_t)b * img_bytes<MT>();
    const int off = ((st * MT + t) * 64 + 16 * g + r) * 16 + 8 * h;
    *reinterpret_cast<half4*>(blk + off) = hi;
    *reinterpret_cast<half4*>(blk + BB / 2 + off) = lo;
    if (j == 0) *reinterpret_cast<int*>(blk + BB + 4 * m) = e;
}

__device__ __forceinline__ void split8(const float4& a, const float4& b, half8& h, half8& l) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        _Float16 hh, ll;
        split_one(v[j], hh, ll);
        h[j] = hh;
        l[j] = ll;
    }
}

__device__ __forceinline__ float absmax8(float m, const float4& a, const float4& b) {
    m = fmaxf(m, fmaxf(fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)),
                       fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w))));
    return fmaxf(m, fmaxf(fmaxf(__builtin_fabsf(b.x), __builtin_fabsf(b.y)),
                          fmaxf(__builtin_fabsf(b.z), __builtin_fabsf(b.w))));
}

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// WM: how W arrives.  1: fp32 (or binary16) rows 16-byte aligned and
// K % 32 == 0, so every step is two 16-byte buffer loads per lane for fp32
// W, one for binary16 W (lane group g takes k = 8g .. 8g+7).  0: the same rows, loaded element by element with
// bounds checks (block boundaries wait for every load).  2: packed by
// heal_pack_w (normalized rows of [32 hi | 32 res] fp16 per 32-wide k block,
// or hi parts alone for a binary16 weight, rows padded): no split in the
// kernel; lane group g takes k = 8g .. 8g+7 of each step (16 contiguous bytes
// of hi, 16 of res), A's operand order follows, and each output is multiplied
// by 2^-e_w[n], the row exponent of W.  The residual is at its own scale, so
// A_hi.W_res joins A_hi.W_hi in one accumulator.
// WF16: W holds binary16 values, exact in fp16: its residual is zero, so each
// step keeps two products, A_hi.W and A_lo.W (2^-10 applied in the fold).
// AVEC: A rows 16-byte aligned, activation units load as one 16-byte load.
// MT == 1, or INKT: the workgroup stages and splits A itself (A, lda);
// otherwise it copies the block images decode_prep_kernel wrote (Ablk).
// SHIFT (splitting A itself): element (m, k) of A is multiplied by
// 2^-kshift[k] before its block maximum and split.  ONE: plain FP16, the
// A_hi.W_hi product alone.  NWK: waves per workgroup.
// KW (one row tile, a k split of 2 .. 8 chunks): the workgroup is one
// 16-row slice of W and its waves are the slice's chunks (wave w takes chunk
// w, blockDim.x / 64 of them), each with its own LDS buffers and no barrier
// in the main loop; the chunk sums meet in LDS and are added in chunk order,
// as the cross-workgroup completion adds them: the same bits, with no
// memory round trips after the main loop.
template <int MT, int WM, bool WF16, bool AVEC, bool SHIFT, bool ONE, int NWK, bool INKT, bool KW = false>
__global__ __launch_bounds__(64 * NWK) void gemm_decode_kernel(const float* __restrict__ A, int64_t lda,
                                                          const unsigned char* __restrict__ Ablk,
                                                          uint32_t a_total_bytes, const void* __restrict__ W,
                                                          int64_t wrow_bytes, const int* __restrict__ wexp,
                                                          float* __restrict__ C, int64_t ldc,
                                                          float* __restrict__ part,
                                                          unsigned long long* __restrict__ flag_base, uint64_t epoch,
                                                          int M, int N, int K, int kchunk,
                                                          const int8_t* __restrict__ kshift,
                                                          uint32_t* __restrict__ status) {
    constexpr bool INK = MT == 1 || INKT;           // split the activation in the kernel
    static_assert(!SHIFT || INK, "with copied blocks the shift is applied by decode_prep_kernel");
    constexpr bool VEC = WM >= 1;
    constexpr bool PKW = WM == 2;                   // W packed: k = 8g .. 8g+7 per lane group
    // k = 8g .. 8g+7 per lane group for every vector-loaded W
    constexpr bool K8 = WM >= 1;
    constexpr int BB = block_bytes<MT>();
    constexpr int SB = img_bytes<MT>();             // LDS bytes per block buffer: planes + exponents
    static_assert(NWK == NW || (NWK == 2 * NW && (MT > 1 || KW)), "8 waves only with several row tiles");
    static_assert(!KW || (MT == 1 && !SHIFT), "chunks as waves with one row tile, no channel shifts");
    constexpr int DMA_PER_WAVE = BB / 1024 / NWK;   // 1 KB per wave-wide direct-to-LDS load
    extern __shared__ __attribute__((aligned(16))) unsigned char sa[];   // 2 x SB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int n0 = KW ? blockIdx.x * ROWS_PER_WAVE : blockIdx.x * (NWK * ROWS_PER_WAVE) + wave * ROWS_PER_WAVE;
    const int n = n0 + (lane & 15);
    const bool row_ok = n < N;
    const int split = KW ? wave : blockIdx.y;
    const int nchunks = KW ? (int)(blockDim.x >> 6) : (int)gridDim.y;   // the plan's k chunks
    const int k_begin = split * kchunk;
    const int k_end = min(k_begin + kchunk, K);
    const int nsteps = (k_end - k_begin + 31) / 32;
    const int nblocks = (nsteps + STEPS - 1) / STEPS;
    // With few chunks (under 8), the chunk's k blocks are visited in a
    // rotated order, rot = (128-row group of W) mod nblocks: workgroups that
    // run together then read at different k offsets, which spreads rows with
    // a power-of-two stride (K = 4096 fp32 rows are 16 KiB apart) over the
    // HBM channels.  With 8 chunks or more their start offsets spread the
    // reads, and rotation measured slower (K = 4096, N = 4096: 24.0 -> 26.1 us
    // at M = 1; K = 4096, N = 14336 with 2 chunks: 55.7 -> 52.0 us), except
    // for rows a multiple of 32 KiB apart read in chunks of 8 blocks or more
    // (K = 8192, N = 4096: 50.2 -> 35.9 us; K = 16384: 67.7 -> 54.8 us).  The
    // order depends on the output rows, (N, K) and W's row stride only, not
    // on M or the workgroup shape.
    const bool rotate = nchunks < 8 || (wrow_bytes % 32768 == 0 && kchunk >= 8 * KA);
    const int rgroup = KW ? blockIdx.x / 8 : blockIdx.x * NWK / 8;   // 128-row group of W
    const int rot = rotate ? (int)((unsigned)rgroup % (unsigned)nblocks) : 0;
    auto pblock = [&](int b) { return b + rot >= nblocks ? b + rot - nblocks : b + rot; };
    // the step to load for logical step L (clamped: the ring's last loads
    // re-read a valid step)
    auto pstep = [&](int L) {
        L = min(L, nblocks * STEPS - 1);
        return min(pblock(L / STEPS) * STEPS + L % STEPS, nsteps - 1);
    };

    // ---- INK: activation blocks split in the kernel.  Wave w owns rows
    //      4 (w RND + j) .. +3 for j < RND (the 16 MT rows shared by the NWK
    //      waves); lane l's unit (j, i) (i < 2) is 4 consecutive k of row
    //      m = 4 (w RND + j) + l % 4 at k = 128 b + 32 s + 16 half + 4 gg with
    //      gg = (l / 4) % 4, half = (l / 16) % 2, s = (l / 32) % 2 + 2 i (for
    //      a packed W: 8 gg + 4 half).  Its hi and lo halves go to the 16-byte
    //      operand slot (s, tile m / 16, lane 16 gg + m % 16), bytes 8 half ..
    //      8 half + 7, of the hi and lo planes; the row's block exponent to
    //      byte BB + 4 m.
    // (KW: each wave stages all 16 rows of its own chunk's blocks)
    constexpr int RND = INK ? (KW ? 4 : 16 * MT / (4 * NWK)) : 1;
    static_assert(!INK || KW || RND * 4 * NWK == 16 * MT, "whole groups of 4 rows per wave");
    const int wbase = KW ? wave * 2 * SB : 0;   // the wave's own LDS buffers (KW)
    float4 areg[RND][2];
    int sreg[2][4];        // SHIFT: the units' 2^-kshift exponents (k >= K reads 0)
    // rows >= M fall outside the resource and read as zero; k past the
    // chunk end is zeroed when the block is stored
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A, (uint32_t)((int64_t)M * lda * 4));
    const __amdgpu_buffer_rsrc_t ksrc = make_rsrc(kshift, SHIFT ? (uint32_t)K : 0u);
    auto urow = [&](int j) { return 4 * ((KW ? 0 : wave * RND) + j) + (lane & 3); };
    const int ugg = (lane >> 2) & 3, uhalf = (lane >> 4) & 1, ust = (lane >> 5) & 1;
    auto unit_k = [&](int pb, int i) {   // pb: the block's place in the chunk
        return k_begin + KA * pb + 32 * (ust + 2 * i) + (K8 ? 8 * ugg + 4 * uhalf : 16 * uhalf + 4 * ugg);
    };
    auto load_a = [&](int b) {
        const int pb = pblock(b);
        if constexpr (SHIFT) {   // the same k for every row group
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t k0 = (uint32_t)unit_k(pb, i);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sreg[i][q] = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(ksrc, k0 + q, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < RND; ++j)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t off = (uint32_t)(((int64_t)urow(j) * lda + unit_k(pb, i)) * 4);
                if (KW && 4 * j >= M) {   // a group of rows past M: zeros, no loads
                    areg[j][i] = make_float4(0.f, 0.f, 0.f, 0.f);
                } else if constexpr (AVEC) {
                    areg[j][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0, 0));
                } else {
                    areg[j][i] = make_float4(
                        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off, 0, 0)),
                        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off + 4, 0, 0)),
                        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off + 8, 0, 0)),
                        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off + 12, 0, 0)));
                }
            }
    };
    auto store_a = [&](int b) {
        unsigned char* base = sa + wbase + (b & 1) * SB;
        const int pb = pblock(b);
#pragma unroll
        for (int j = 0; j < RND; ++j) {
            float v[2][4];
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int k = unit_k(pb, i);
                const float x[4] = {areg[j][i].x, areg[j][i].y, areg[j][i].z, areg[j][i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[i][q] = k + q < k_end ? (SHIFT ? __builtin_ldexpf(x[q], -sreg[i][q]) : x[q]) : 0.0f;
                    mx = fmaxf(mx, __builtin_fabsf(v[i][q]));
                }
            }
            // the row's maximum over the block: the 16 lanes with the same l % 4
            mx = max16_mod4(mx);
            const int e = row_norm_exp(mx);
            const int m = urow(j), t = m >> 4, r = m & 15;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                half4 h, l;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    _Float16 hh, ll;
                    split_one(__builtin_ldexpf(v[i][q], e), hh, ll);
                    h[q] = hh;
                    l[q] = ll;
                }
                const int off = (((ust + 2 * i) * MT + t) * 64 + 16 * ugg + r) * 16 + 8 * uhalf;
                *reinterpret_cast<half4*>(base + off) = h;
                *reinterpret_cast<half4*>(base + BB / 2 + off) = l;
            }
            if ((lane >> 2) == 0) *reinterpret_cast<int*>(base + BB + 4 * m) = e;
        }
    };

    // block images (MT > 1): wave w copies 1 KB pieces w, w + NWK, ... of the
    // planes; wave 0 also the 256 bytes of exponents (4 bytes per lane)
    const int blk0 = k_begin / KA;
    const __amdgpu_buffer_rsrc_t pbrsrc = make_rsrc(Ablk, a_total_bytes);
    auto dma_block = [&](int b) {
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            const int piece = wave + NWK * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pbrsrc, (lds_ptr)(sa + (b & 1) * SB + piece * 1024), 16,
                                                     (uint32_t)(lane * 16),
                                                     (uint32_t)(blk0 + pblock(b)) * (uint32_t)SB + piece * 1024u, 0, 0);
        }
        if (wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pbrsrc, (lds_ptr)(sa + (b & 1) * SB + BB), 4,
                                                     (uint32_t)(lane * 4), (uint32_t)(blk0 + pblock(b)) * (uint32_t)SB + BB,
                                                     0, 0);
    };

    // W: lane reads row n, k = k_begin + 32 step + 8g .. 8g+7 (element loads:
    // {4g.., 16+4g..}) (scalars made explicit: the buffer resource must live in SGPRs)
    constexpr int ESZ = WF16 ? 2 : 4;          // bytes per W element (unpacked)
    constexpr int KBB = WF16 ? 64 : 128;       // packed bytes per row and 32-wide k block
    constexpr int PFW = PF;                    // W steps in flight
    constexpr int LPS = K8 && WF16 ? 1 : 2;    // buffer loads per W step (VEC)
    using WReg = std::conditional_t<WF16, u32x4, u32x8>;   // one step's 8 W values (packed: hi, then res)
    const int64_t ldw = wrow_bytes / ESZ;      // unpacked: elements per row
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(ROWS_PER_WAVE, N - n0)));
    const int wrow0 = __builtin_amdgcn_readfirstlane(min(n0, N - 1));
    const unsigned char* Wb = static_cast<const unsigned char*>(W);
    const __amdgpu_buffer_rsrc_t wrsrc =
        make_rsrc(Wb + (int64_t)wrow0 * wrow_bytes, (uint32_t)((int64_t)nrows * wrow_bytes));
    const uint32_t wlane = PKW ? (uint32_t)((lane & 15) * wrow_bytes + (int64_t)(k_begin / 32) * KBB + 16 * g)
                               : (uint32_t)((lane & 15) * wrow_bytes + (int64_t)(k_begin + (K8 ? 8 : 4) * g) * ESZ);
    auto load_w = [&](int step, WReg& w) {
        if constexpr (PKW) {
            const uint32_t off = wlane + (uint32_t)(step * KBB);
            const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0);
            if constexpr (WF16) {
                w = h;
            } else {
                const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off + 64, 0, 0);
                w = WReg{h[0], h[1], h[2], h[3], r[0], r[1], r[2], r[3]};
            }
        } else if (VEC) {
            const uint32_t off = wlane + (uint32_t)(step * 32 * ESZ);
            if constexpr (WF16) {
                w = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0);
            } else {
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0);
                const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off + 4 * ESZ, 0, 0);
                w = WReg{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            }
        } else {
            const int ka = k_begin + 32 * step + 4 * g, kb = ka + 16;
            if constexpr (WF16) {
                const uint16_t* wrow = static_cast<const uint16_t*>(W) + (int64_t)(row_ok ? n : 0) * ldw;
                uint32_t t[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t[j] = (row_ok && ka + j < k_end) ? wrow[ka + j] : 0u;
                    t[4 + j] = (row_ok && kb + j < k_end) ? wrow[kb + j] : 0u;
                }
                w = WReg{t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16), t[6] | (t[7] << 16)};
            } else {
                const float* wrow = static_cast<const float*>(W) + (int64_t)(row_ok ? n : 0) * ldw;
                float t[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t[j] = (row_ok && ka + j < k_end) ? wrow[ka + j] : 0.f;
                    t[4 + j] = (row_ok && kb + j < k_end) ? wrow[kb + j] : 0.f;
                }
                w = __builtin_bit_cast(WReg, (floatx8){t[0], t[1], t[2], t[3], t[4], t[5], t[6], t[7]});
            }
        }
    };

    // running sums (fp32) and one block's accumulators
    float tot[MT][4];
    floatx4 acc_hh[MT], acc_c[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) tot[t][e] = 0.f;

    // prologue: W for steps 0 .. PFW-1 and activation block 0 in flight
    // together; block 0 lands in LDS buffer 0 (split here, or copied); its
    // loads are issued first, so that waiting for them leaves W in flight
    // (issuing the activation loads last cost 0.7-1.1 us per call on the
    // in-kernel split path)
    WReg wr[PFW];
    if constexpr (INK) {
        load_a(0);   // first, so that waiting for it leaves W in flight
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < PFW; ++s) load_w(pstep(s), wr[s]);
        __builtin_amdgcn_sched_barrier(0);
        store_a(0);
        __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    } else {
        dma_block(0);
#pragma unroll
        for (int s = 0; s < PFW; ++s) load_w(pstep(s), wr[s]);
        __builtin_amdgcn_sched_barrier(0);
        if (VEC) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS * PFW));   // block 0 landed; W still in flight
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    if constexpr (!KW) __builtin_amdgcn_s_barrier();   // KW: the wave's own buffers, LDS in program order
    __builtin_amdgcn_sched_barrier(0);
    float wmax = 0.0f;

    // one activation block of STEPS steps; J = position of its first step
    // in the PFW-deep W register ring
    auto run_block = [&](int b, auto J_) {
        constexpr int J = decltype(J_)::value;
        const bool more = b + 1 < nblocks;
        if (more) {                            // next activation block, in flight during this one
            if constexpr (INK) load_a(b + 1);
            else dma_block(b + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* abuf = sa + wbase + (b & 1) * SB;
        const int pb = pblock(b);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) { acc_hh[t][e] = 0.f; acc_c[t][e] = 0.f; }
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int step = b * STEPS + s;
            WReg& w = wr[J + s];
            half8 wh, wl;
            if constexpr (WF16) {
                wh = __builtin_bit_cast(half8, w);
            } else if constexpr (PKW) {
                wh = __builtin_bit_cast(half8, (u32x4){w[0], w[1], w[2], w[3]});
                wl = __builtin_bit_cast(half8, (u32x4){w[4], w[5], w[6], w[7]});
            } else {
                const floatx8 wf = __builtin_bit_cast(floatx8, w);
                const float4 ra = {wf[0], wf[1], wf[2], wf[3]}, rb = {wf[4], wf[5], wf[6], wf[7]};
                split8(ra, rb, wh, wl);
                wmax = absmax8(wmax, ra, rb);
            }
            load_w(pstep(step + PFW), w);
            if (pb * STEPS + s < nsteps) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int off = ((s * MT + t) * 64 + lane) * 16;
                    const half8 ah = *reinterpret_cast<const half8*>(abuf + off);
                    const half8 al = *reinterpret_cast<const half8*>(abuf + BB / 2 + off);
                    mfma16(ah, wh, acc_hh[t]);
                    if constexpr (!WF16 && !ONE) mfma16(ah, wl, PKW ? acc_hh[t] : acc_c[t]);   // packed: res unshifted
                    if constexpr (!ONE) mfma16(al, wh, acc_c[t]);
                }
            }
        }
        // fold the block: rows t*16 + 4g + e of this lane, scaled by their
        // block exponents 2^-e
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int4 er = *reinterpret_cast<const int4*>(abuf + BB + 4 * (t * 16 + 4 * g));
            const int ev[4] = {er.x, er.y, er.z, er.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                tot[t][e] += __builtin_ldexpf(acc_hh[t][e] + acc_c[t][e] * 0.0009765625f, -ev[e]);
        }
        if (more) {
            // the other buffer was last read in block b - 1, before the
            // previous barrier; it now holds (or receives) block b + 1
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (INK) {
                store_a(b + 1);
                __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
            } else {
                // the copy was issued before this block's LPS * STEPS W loads
                if (VEC) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPS * STEPS));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            if constexpr (!KW) __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    static_assert(PFW % STEPS == 0 && PFW / STEPS <= 4, "W ring of whole blocks");
    // a do-while (every chunk has at least one block): the prologue's loads
    // then stay in the entry block instead of being sunk into the loop
    int b = 0;
    do {
        run_block(b, std::integral_constant<int, 0>{});
        if constexpr (PFW / STEPS > 1)
            if (b + 1 < nblocks) run_block(b + 1, std::integral_constant<int, STEPS>{});
        if constexpr (PFW / STEPS > 2)
            if (b + 2 < nblocks) run_block(b + 2, std::integral_constant<int, 2 * STEPS>{});
        if constexpr (PFW / STEPS > 3)
            if (b + 3 < nblocks) run_block(b + 3, std::integral_constant<int, 3 * STEPS>{});
        b += PFW / STEPS;
    } while (b < nblocks);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // drain the clamped tail loads
    // the normalized activation cannot overflow fp16; W is split as it is
    if (status && __builtin_amdgcn_ballot_w64(wmax >= 65520.0f) && lane == 0)
        atomicOr(status, (uint32_t)HEAL_FLAG_F16_RANGE);

    // ---- epilogue: lane holds column n, rows t*16 + 4g + e ------------------
    if constexpr (PKW) {   // W's row exponent (padding rows hold 0)
        const int ew = row_ok ? wexp[n] : 0;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) tot[t][e] = __builtin_ldexpf(tot[t][e], -ew);
    }
    if constexpr (KW) {
        // each wave's chunk sums into its own (no longer read) LDS buffer;
        // after the one barrier every wave reaches, wave 0 adds them in
        // chunk order and writes C
        float* mine = reinterpret_cast<float*>(sa + wbase);
        *reinterpret_cast<float4*>(mine + 4 * lane) = make_float4(tot[0][0], tot[0][1], tot[0][2], tot[0][3]);
        __syncthreads();
        if (wave != 0 || !row_ok) return;
        float acc[4] = {tot[0][0], tot[0][1], tot[0][2], tot[0][3]};
        for (int c = 1; c < nchunks; ++c) {
            const float4 p = *reinterpret_cast<const float4*>(sa + c * 2 * SB + 16 * lane);
            acc[0] += p.x;
            acc[1] += p.y;
            acc[2] += p.z;
            acc[3] += p.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * g + e;
            if (m < M) C[(int64_t)m * ldc + n] = acc[e];
        }
        return;
    }
    const int nsplit = gridDim.y;
    if (nsplit == 1) {
        if (!row_ok) return;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = t * 16 + 4 * g + e;
                if (m < M) C[(int64_t)m * ldc + n] = tot[t][e];
            }
        return;
    }
    // split-K: this chunk's partials P[split][m][n], stored through to memory
    // (write-through: no dirty L2 line to write back), completed before the
    // workgroup counts itself in on its row block's counter
    const int64_t pstride = (int64_t)M * N;
    if (row_ok) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = t * 16 + 4 * g + e;
                if (m < M)
                    __hip_atomic_store(part + split * pstride + (int64_t)m * N + n, tot[t][e], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __shared__ int missing;
    if (tid == 0) missing = 0;
    __syncthreads();
    if (epoch == 0) {
        // counter form (a zeroed array of one counter per row block, which
        // every call leaves zeroed: the same arguments can be replayed, as
        // from a captured graph): the workgroup counts itself in once its
        // partials are stored; the one that counts last sums and puts the
        // counter back to zero
        if (tid == 0) {
            unsigned long long* cnt = flag_base + blockIdx.x;
            const unsigned long long old =
                __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == (unsigned long long)nsplit)
                __hip_atomic_store(cnt, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                missing = 1;
        }
    } else {
        // epoch form: the workgroup's flag for (row block, chunk) := this
        // call's epoch, also written through and completed; then it reads the
        // flags of all chunks of its row block.  The workgroup whose flag
        // completes last sees every flag set, so at least one workgroup sums;
        // any other that sees them all too writes the same values.  A flag
        // from an earlier call (or whatever the workspace held) differs from
        // this call's epoch.
        unsigned long long* flags = flag_base + (int64_t)blockIdx.x * nsplit;
        if (tid == 0) {
            __hip_atomic_store(flags + split, (unsigned long long)epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __syncthreads();
        bool miss = false;
        for (int j = tid; j < nsplit; j += 64 * NWK)
            miss |= __hip_atomic_load(flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
                    (unsigned long long)epoch;
        if (__builtin_amdgcn_ballot_w64(miss) && lane == 0) missing = 1;
    }
    __syncthreads();
    if (missing || !row_ok) return;
    // a workgroup that saw every chunk done: C = sum over chunks in chunk order
    // (the other chunks' partials read past the L2, its own from registers);
    // the loads of NB chunks for all the lane's outputs are in flight together
    constexpr int NB = 16 / MT;
    float acc[MT][4];
    for (int s0 = 0; s0 < nsplit; s0 += NB) {
        float pv[NB][MT][4];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int sj = min(s0 + j, nsplit - 1);
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = min(t * 16 + 4 * g + e, M - 1);
                    pv[j][t][e] = sj == split ? tot[t][e]
                                              : __hip_atomic_load(part + sj * pstride + (int64_t)m * N + n,
                                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (s0 + j < nsplit)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[t][e] = (s0 + j == 0) ? pv[j][t][e] : acc[t][e] + pv[j][t][e];
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = t * 16 + 4 * g + e;
            if (m < M) C[(int64_t)m * ldc + n] = acc[t][e];
        }
}

int mtiles(int64_t M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

}  // namespace

// workspace: split-K flags, activation block images, split-K partials
int64_t DecodePlan::bytes() const {
    return (c_bytes + 255) / 256 * 256 + (a_bytes + 255) / 256 * 256 + (p_bytes + 255) / 256 * 256;
}

bool decode_chunks_as_waves(int64_t M, int64_t N, const DecodePlan& p, bool kshift) {
    const int64_t nslices = (N + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    return mtiles(M) == 1 && !kshift && p.splits >= 2 && p.splits <= 2 * NW && p.kchunk <= 4 * KA && nslices >= 256;
}

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K) {
    DecodePlan p{};
    const int64_t nblk = (N + DEC_ROWS - 1) / DEC_ROWS;
    const int64_t kblocks = std::max<int64_t>(1, (K + 255) / 256);
    // about TARGET_WG workgroups in one round, without going over
    int64_t want = std::max<int64_t>(1, TARGET_WG / std::max<int64_t>(nblk, 1));
    want = std::min(want, kblocks);
    const int64_t per = (K + want - 1) / want;
    p.kchunk = std::max<int64_t>(256, (per + 255) / 256 * 256);
    p.splits = (int)std::max<int64_t>(1, (K + p.kchunk - 1) / p.kchunk);
    const int64_t ablocks = (K + KA - 1) / KA;
    const int mt = mtiles(M);
    p.a_bytes = mt == 1 ? 0 : ablocks * (mt == 2 ? img_bytes<2>() : img_bytes<4>());
    p.p_bytes = p.splits > 1 ? (p.splits * M * N * 4 + 255) / 256 * 256 : 0;
    p.ncount = p.splits > 1 ? (N + DEC_ROWS - 1) / DEC_ROWS * p.splits : 0;   // (row block, chunk) flags
    p.c_bytes = p.ncount * 8;
    return p;
}

hipError_t launch_gemm_decode(const float* A, int64_t lda, const int8_t* kshift, const void* W, bool wf16,
                              bool packed, bool one, int64_t ldw, float* C, int64_t ldc, int64_t M, int64_t N,
                              int64_t K, void* workspace, const DecodePlan& plan, uint64_t epoch,
                              unsigned long long* counters, uint32_t* status, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M > 64 || K == 0 || (!counters && epoch == 0)) return hipErrorInvalidValue;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    // split-K completion: the epoch flags at the start of the workspace, or
    // the caller's zeroed counters (epoch 0 selects them in the kernel)
    unsigned long long* flags = counters ? counters : reinterpret_cast<unsigned long long*>(ws);
    if (counters) epoch = 0;
    unsigned char* ablk = ws + (plan.c_bytes + 255) / 256 * 256;
    float* part = reinterpret_cast<float*>(ablk + (plan.a_bytes + 255) / 256 * 256);
    const int nablk = (int)((K + KA - 1) / KA);
    const int mt = mtiles(M);
    const int64_t nblk2 = (N + 2 * DEC_ROWS - 1) / (2 * DEC_ROWS);
    const bool wide = mt > 1 && nblk2 * plan.splits >= (mt == 4 ? WIDE_MIN_WG4 : WIDE_MIN_WG2);
    const int wg_rows = (wide ? 2 * NW : NW) * ROWS_PER_WAVE;
    const dim3 grid((unsigned)((N + wg_rows - 1) / wg_rows), (unsigned)plan.splits);
    // W loads of 8 elements per step (two 16-byte loads of fp32, one of
    // binary16) need 16-byte aligned rows and whole k32 steps
    const bool vec = (reinterpret_cast<uintptr_t>(W) & 15) == 0 && (ldw & (wf16 ? 7 : 3)) == 0 && (K & 31) == 0;
    // the activation's k order within a step: 8 consecutive k per lane group
    // for every vector-loaded W
    const bool k8 = packed || vec;
    // packed W: padded rows, the row exponents after them
    const int64_t wrow_bytes = packed ? (wf16 ? pack_row_bytes_hi(K) : pack_row_bytes(K)) : ldw * (wf16 ? 2 : 4);
    const int* wexp = packed ? reinterpret_cast<const int*>(static_cast<const unsigned char*>(W) +
                                                            (wf16 ? pack_data_bytes_hi(N, K) : pack_data_bytes(N, K)))
                             : nullptr;
    // activation units load as float4 when rows are 16-byte aligned
    const bool avec = (reinterpret_cast<uintptr_t>(A) & 15) == 0 && (lda & 3) == 0;
    // With several row tiles the workgroups split their activation blocks
    // themselves (no block images, no first kernel) when that work is light:
    // one group of 4 rows per wave, or two over short chunks (at most 4
    // blocks).  Measured (K, N, M = 32 / 64): it gains 1.4 - 4.1 us on those
    // shapes, and loses 1.3 - 22 us with 2 groups over 14 - 16 blocks or 4
    // groups per wave.  Both forms store the same split blocks: the results
    // are identical.
    const int rnd = 16 * mt / (4 * (wide ? 2 * NW : NW));
    // One row tile, 2 .. 8 chunks of at most 4 blocks, and at least 256
    // slices of 16 rows (one workgroup per slice fills the chip): the chunks
    // are the waves of one workgroup (KW), with no completion through memory.
    // Measured per call (back to back, cold Infinity Cache): K = N = 4096
    // (8 chunks of 4 blocks) 21.7 -> 19.5 us at M = 1, 22.4 -> 20.8 us at
    // M = 8; with longer chunks the chunk-per-wave grid streams slower than
    // it saves (K = 14336, N = 4096, 8 chunks of 14 blocks: 47.8 -> 47.9 us
    // at M = 1, 49.2 -> 53.2 us at M = 8; K = 4096, N = 14336, 2 chunks of
    // 16 blocks: 51.7 -> 52.6 and 52.5 -> 57.0 us), so it stays off there.
    // (Not with a_kshift: that form's per-wave staging of all 16 rows did not
    // fit in registers.)
    const int64_t nslices = (N + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
    const bool kw = decode_chunks_as_waves(M, N, plan, kshift != nullptr);
    const bool ink = mt > 1 && !kshift && avec && (rnd == 1 || (rnd == 2 && plan.kchunk / KA <= 4));
#define HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW_, INK_)                                \
    hipLaunchKernelGGL((gemm_decode_kernel<MT_, VEC_, F16_, AV_, SH_, ONE_, NW_, INK_>), grid, dim3(64 * NW_), \
                       2 * img_bytes<MT_>(), s, A, lda, ablk, (uint32_t)plan.a_bytes, W, wrow_bytes, wexp, C, ldc, part, \
                       flags, epoch,                                                                          \
                       (int)M, (int)N, (int)K, (int)plan.kchunk, kshift, status)
#define HEAL_DEC_LAUNCH_INK(MT_, VEC_, F16_, AV_, SH_, ONE_, NW_)                                      \
    do {                                                                                                \
        if constexpr (AV_ && !SH_) {                                                                    \
            if (ink) {                                                                                  \
                HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW_, true);                         \
                break;                                                                                  \
            }                                                                                           \
        }                                                                                               \
        HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW_, false);                                \
    } while (0)
#define HEAL_DEC_LAUNCH_KW(VEC_, F16_, AV_, SH_, ONE_)                                                 \
    hipLaunchKernelGGL((gemm_decode_kernel<1, VEC_, F16_, AV_, SH_, ONE_, 2 * NW, false, true>),          \
                       dim3((unsigned)nslices), dim3(64 * plan.splits), plan.splits * 2 * img_bytes<1>(), s, A, \
                       lda, ablk, (uint32_t)plan.a_bytes, W, wrow_bytes, wexp, C, ldc, part, flags, epoch,    \
                       (int)M, (int)N, (int)K, (int)plan.kchunk, kshift, status)
#define HEAL_DEC_LAUNCH(MT_, VEC_, F16_, AV_, SH_, ONE_)                                                \
    do {                                                                                                \
        if constexpr (MT_ > 1) {                                                                        \
            if (wide) HEAL_DEC_LAUNCH_INK(MT_, VEC_, F16_, AV_, SH_, ONE_, 2 * NW);                     \
            else HEAL_DEC_LAUNCH_INK(MT_, VEC_, F16_, AV_, SH_, ONE_, NW);                              \
        } else {                                                                                        \
            if constexpr (!SH_) {                                                                       \
                if (kw) {                                                                               \
                    HEAL_DEC_LAUNCH_KW(VEC_, F16_, AV_, false, ONE_);                                   \
                    break;                                                                              \
                }                                                                                       \
            }                                                                                           \
            HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW, false);                             \
        }                                                                                               \
    } while (0)
#define HEAL_DEC_MAIN(MT_, VEC_, F16_, AV_, SH_)                                                        \
    do {                                                                                                \
        if (one) HEAL_DEC_LAUNCH(MT_, VEC_, F16_, AV_, SH_, true);                                      \
        else HEAL_DEC_LAUNCH(MT_, VEC_, F16_, AV_, SH_, false);                                         \
    } while (0)
#define HEAL_DEC_AV(MT_, VEC_, F16_, SH_)                                                               \
    do {                                                                                                \
        if (avec) HEAL_DEC_MAIN(MT_, VEC_, F16_, true, SH_);                                            \
        else HEAL_DEC_MAIN(MT_, VEC_, F16_, false, SH_);                                                \
    } while (0)
#define HEAL_DEC(MT_, SH_)                                                                              \
    do {                                                                                                \
        if constexpr ((MT_) > 1) {                                                                      \
          if (!ink) {                                                                                   \
            const dim3 pgrid(16 * (MT_), (unsigned)((nablk * 32 + PREP_T - 1) / PREP_T));                \
            if (avec && k8)                                                                             \
                hipLaunchKernelGGL((decode_prep_kernel<MT_, true, true>), pgrid, dim3(PREP_T), 0, s, A, lda, \
                                   (int)M, (int)K, nablk, kshift, ablk);                                \
            else if (avec)                                                                              \
                hipLaunchKernelGGL((decode_prep_kernel<MT_, true, false>), pgrid, dim3(PREP_T), 0, s, A, lda, \
                                   (int)M, (int)K, nablk, kshift, ablk);                                \
            else if (k8)                                                                                \
                hipLaunchKernelGGL((decode_prep_kernel<MT_, false, true>), pgrid, dim3(PREP_T), 0, s, A, lda, \
                                   (int)M, (int)K, nablk, kshift, ablk);                                \
            else                                                                                        \
                hipLaunchKernelGGL((decode_prep_kernel<MT_, false, false>), pgrid, dim3(PREP_T), 0, s, A, lda, \
                                   (int)M, (int)K, nablk, kshift, ablk);                                \
          }                                                                                             \
        }                                                                                               \
        if (wf16) {                                                                                     \
            if (packed) HEAL_DEC_AV(MT_, 2, true, SH_);                                                 \
            else if (vec) HEAL_DEC_AV(MT_, 1, true, SH_);                                               \
            else HEAL_DEC_AV(MT_, 0, true, SH_);                                                        \
        } else {                                                                                        \
            if (packed) HEAL_DEC_AV(MT_, 2, false, SH_);                                                \
            else if (vec) HEAL_DEC_AV(MT_, 1, false, SH_);                                              \
            else HEAL_DEC_AV(MT_, 0, false, SH_);                                                       \
        }                                                                                               \
    } while (0)
    if (mt == 1) {
        if (kshift) HEAL_DEC(1, true);
        else HEAL_DEC(1, false);
    } else if (mt == 2) {
        HEAL_DEC(2, false);
    } else {
        HEAL_DEC(4, false);
    }
#undef HEAL_DEC
#undef HEAL_DEC_AV
#undef HEAL_DEC_MAIN
#undef HEAL_DEC_LAUNCH
#undef HEAL_DEC_LAUNCH_INK
#undef HEAL_DEC_LAUNCH_KW
#undef HEAL_DEC_LAUNCH_NW
    return hipGetLastError();
}

}  // namespace heal

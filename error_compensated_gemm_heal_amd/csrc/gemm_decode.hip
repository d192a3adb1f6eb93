// Decode-shaped FP32-accurate GEMM (M <= 64) on gfx950 16-bit MFMA.
//
// Same arithmetic as the prefill kernel (HEAL paper, section 3, "Mitigating
// GEMM Truncation via FP16 Promotion and Algebraic Compensation"):
//     C = A_hi.B_hi + 2^-10 (A_hi.B_lo + A_lo.B_hi),  fp32 accumulation,
// but shaped for a skinny activation, where the weight is the traffic:
//  * W is read once from HBM as fp32 [N, K] (4 bytes per element, the same
//    bytes as its two fp16 parts) and split into hi/lo in registers;
//  * FP16's narrow range (the same paragraph: handled by targeted
//    rescaling): a small first kernel (decode_prep_kernel, one workgroup per
//    activation row) finds each row's largest magnitude and the power of two
//    2^e that puts it in [2^14, 2^15); rows are split as x 2^e and each
//    output is multiplied back by 2^-e in fp32, so the result does not
//    depend on the activation's absolute scale (W is split as it is);
//  * the activation (<= 64 rows) is staged in 128-wide k blocks in a
//    double-buffered LDS tile, in MFMA operand order, so every operand read
//    is one conflict-free 16-byte LDS access.  Up to 16 rows, each
//    workgroup loads the next block into registers while the current one
//    is in use and normalizes and splits it itself; above 16 rows, where that
//    split would be repeated by every workgroup, the first kernel also writes
//    the split rows as operand-ordered planes and workgroups copy blocks of
//    them into LDS with direct-to-LDS loads;
//  * v_mfma_f32_16x16x32_f16 with the activation as the 16-row operand and W
//    as the 16-column operand (16 W rows per wave), so output columns are
//    consecutive lanes;
//  * inside each 32-wide k step, lane group g (lanes 16g..16g+15) carries
//    k = 4g..4g+3 and 16+4g..16+4g+3: any k order is valid as long as both
//    operands use it, and this one makes each W load a 64-byte run per row;
//  * W for the next 8 k steps is always in flight: every step issues exactly
//    two W loads (the last steps re-read a clamped step), so the number of
//    loads outstanding at each block boundary is a constant;
//  * split-K: the k range is cut into chunks chosen from (N, K) only, and
//    chunk partials are summed in chunk order by a second kernel.  The
//    summation order of an output therefore does not depend on M: a
//    decode-sized product does not change with the batch it is computed in.
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

// ---- the first kernel: row exponents and (MT > 1) operand-ordered planes ----
// Workgroup m (one per row of the MT 16-row tiles) takes row m of A: its
// largest magnitude (after the optional 2^-kshift[k]) gives the row exponent
// e_m (aexp[m]; rows >= M get 0).  With MT > 1 it then writes the row's
// split, x 2^(e_m - kshift[k]) as hi = fp16, lo = fp16((x - hi) 2^10), in
// operand order: block b (k in [128 b, 128 b + 128)), plane p (0 = hi,
// 1 = lo), step s, tile t, lane l = 16 g + r holds, as 8 fp16, row 16 t + r
// at k = 128 b + 32 s + {4g .. 4g+3, 16+4g .. 16+4g+3}.  Rows >= M and
// k >= K are zero.
template <int MT>
__global__ __launch_bounds__(256) void decode_prep_kernel(const float* __restrict__ A, int64_t lda, int M, int K,
                                                          int nblk, const int8_t* __restrict__ kshift,
                                                          int* __restrict__ aexp, unsigned char* __restrict__ out) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const float* a = A + (int64_t)m * lda;
    auto shift = [&](int k) { return kshift ? -(int)kshift[k] : 0; };
    float mx = 0.0f;
    for (int k = tid; k < K && m < M; k += 256) mx = fmaxf(mx, __builtin_fabsf(__builtin_ldexpf(a[k], shift(k))));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = row_norm_exp(mx);
    if (tid == 0) aexp[m] = e;
    if constexpr (MT > 1) {
        const int t = m >> 4, r = m & 15;
        for (int item = tid; item < nblk * STEPS * 4; item += 256) {   // (b, s, g)
            const int g = item & 3, st = (item >> 2) % STEPS, b = item / (4 * STEPS);
            const int k0 = b * KA + 32 * st;
            half8 h, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int k = k0 + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
                _Float16 hh, ll;
                // one scaling by 2^(e - kshift[k]), as the in-kernel split does
                split_one((m < M && k < K) ? __builtin_ldexpf(a[k], e + shift(k)) : 0.0f, hh, ll);
                h[j] = hh;
                lo[j] = ll;
            }
            unsigned char* blk = out + (int64_t)b * block_bytes<MT>();
            const int off = ((st * MT + t) * 64 + 16 * g + r) * 16;
            *reinterpret_cast<half8*>(blk + off) = h;
            *reinterpret_cast<half8*>(blk + block_bytes<MT>() / 2 + off) = lo;
        }
    }
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

// VEC: W rows aligned to the load width and K % 32 == 0, so every step is two
// buffer loads per lane (16 bytes each for fp32 W, 8 for fp16 W).  Otherwise
// lanes load element by element with bounds checks, and block boundaries
// wait for every load.
// WF16: W holds binary16 values, exact in fp16: its residual is zero, so each
// step keeps two products, A_hi.W and A_lo.W (2^-10 applied at the end).
// AVEC: A rows 16-byte aligned, activation units load as one 16-byte load.
// MT == 1 stages A itself (A, lda); MT > 1 copies the pre-split blocks (Ablk).
// SHIFT (MT == 1): element (m, k) of A is multiplied by 2^-kshift[k] before
// its split.  ONE: plain FP16, the A_hi.W_hi product alone.
template <int MT, bool VEC, bool WF16, bool AVEC, bool SHIFT, bool ONE, int NWK>
__global__ __launch_bounds__(64 * NWK) void gemm_decode_kernel(const float* __restrict__ A, int64_t lda,
                                                          const int* __restrict__ aexp,
                                                          const unsigned char* __restrict__ Ablk,
                                                          int a_total_bytes, const void* __restrict__ W,
                                                          int64_t ldw, float* __restrict__ out, int64_t ldo,
                                                          int64_t split_stride, int M, int N, int K,
                                                          int kchunk, const int8_t* __restrict__ kshift,
                                                          uint32_t* __restrict__ status) {
    static_assert(!SHIFT || MT == 1, "with MT > 1 the shift is applied by decode_prep_kernel");
    constexpr int BB = block_bytes<MT>();
    constexpr bool INK = MT == 1;                   // split the activation in the kernel
    constexpr int AU = 2 * MT;                      // 4-wide activation units per thread per block
    static_assert(NWK == NW || (NWK == 2 * NW && MT > 1), "8 waves only with the copied activation");
    constexpr int DMA_PER_WAVE = BB / 1024 / NWK;   // 1 KB per wave-wide direct-to-LDS load
    extern __shared__ __attribute__((aligned(16))) unsigned char sa[];   // 2 x BB

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int n0 = blockIdx.x * (NWK * ROWS_PER_WAVE) + wave * ROWS_PER_WAVE;
    const int n = n0 + (lane & 15);
    const bool row_ok = n < N;
    const int split = blockIdx.y;
    const int k_begin = split * kchunk;
    const int k_end = min(k_begin + kchunk, K);
    const int nsteps = (k_end - k_begin + 31) / 32;
    const int nblocks = (nsteps + STEPS - 1) / STEPS;

    // ---- activation blocks.  Unit x = tid + 256 i (i < AU) of a block is 4
    //      consecutive k of one row: r = x % 16, g = (x / 16) % 4, half =
    //      (x / 64) % 2, step s = (x / 128) % 4, tile t = x / 512; it holds
    //      row 16 t + r at k = 128 b + 32 s + 16 half + 4 g .. + 3, and its
    //      hi and lo halves go to the 16-byte operand slot (s, t, lane 16 g + r),
    //      bytes 8 half .. 8 half + 7, of the hi and lo planes.
    float4 areg[AU];
    int sreg[AU][4];   // SHIFT: the units' 2^-kshift exponents (k >= K reads 0)
    // rows >= M fall outside the resource and read as zero; k past the
    // chunk end is zeroed when the block is stored
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A, (uint32_t)((int64_t)M * lda * 4));
    const __amdgpu_buffer_rsrc_t ksrc = make_rsrc(kshift, SHIFT ? (uint32_t)K : 0u);
    auto unit_k = [&](int b, int x) {
        return k_begin + KA * b + 32 * ((x >> 7) & 3) + 16 * ((x >> 6) & 1) + 4 * ((x >> 4) & 3);
    };
    auto load_a = [&](int b) {
#pragma unroll
        for (int i = 0; i < AU; ++i) {
            const int x = tid + 256 * i;
            const int m = 16 * (x >> 9) + (x & 15);
            const uint32_t off = (uint32_t)(((int64_t)m * lda + unit_k(b, x)) * 4);
            if constexpr (AVEC) {
                areg[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, off, 0, 0));
            } else {
                areg[i] = make_float4(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off, 0, 0)),
                                      __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off + 4, 0, 0)),
                                      __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off + 8, 0, 0)),
                                      __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(arsrc, off + 12, 0, 0)));
            }
            if constexpr (SHIFT) {
                const uint32_t k0 = (uint32_t)unit_k(b, x);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sreg[i][j] = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(ksrc, k0 + j, 0, 0);
            }
        }
    };
    // MT == 1: the thread's units all lie in row tid % 16; its exponent
    const int erow = INK ? aexp[tid & 15] : 0;
    auto store_a = [&](int b) {
        unsigned char* base = sa + (b & 1) * BB;
#pragma unroll
        for (int i = 0; i < AU; ++i) {
            const int x = tid + 256 * i;
            const int r = x & 15, gg = (x >> 4) & 3, half = (x >> 6) & 1, st = (x >> 7) & 3, t = x >> 9;
            const int k = unit_k(b, x);
            float v[4] = {k < k_end ? areg[i].x : 0.0f, k + 1 < k_end ? areg[i].y : 0.0f,
                          k + 2 < k_end ? areg[i].z : 0.0f, k + 3 < k_end ? areg[i].w : 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __builtin_ldexpf(v[j], SHIFT ? erow - sreg[i][j] : erow);
            half4 h, l;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                _Float16 hh, ll;
                split_one(v[j], hh, ll);
                h[j] = hh;
                l[j] = ll;
            }
            const int off = ((st * MT + t) * 64 + 16 * gg + r) * 16 + 8 * half;
            *reinterpret_cast<half4*>(base + off) = h;
            *reinterpret_cast<half4*>(base + BB / 2 + off) = l;
        }
    };

    // pre-split activation blocks: wave w copies 1 KB pieces w, w + NWK, ...
    const int blk0 = k_begin / KA;
    const __amdgpu_buffer_rsrc_t pbrsrc = make_rsrc(Ablk, (uint32_t)a_total_bytes);
    auto dma_block = [&](int b) {
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i) {
            const int piece = wave + NWK * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(pbrsrc, (lds_ptr)(sa + (b & 1) * BB + piece * 1024), 16,
                                                     (uint32_t)(lane * 16),
                                                     (uint32_t)((blk0 + b) * BB + piece * 1024), 0, 0);
        }
    };

    // W: lane reads row n, k = k_begin + 32 step + {4g.., 16+4g..}
    // (scalars made explicit: the buffer resource must live in SGPRs)
    constexpr int ESZ = WF16 ? 2 : 4;          // bytes per W element
    constexpr int PFW = PF;                    // W steps in flight
    using WReg = std::conditional_t<WF16, u32x4, u32x8>;   // one step's 8 W values
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(ROWS_PER_WAVE, N - n0)));
    const int wrow0 = __builtin_amdgcn_readfirstlane(min(n0, N - 1));
    const unsigned char* Wb = static_cast<const unsigned char*>(W);
    const __amdgpu_buffer_rsrc_t wrsrc =
        make_rsrc(Wb + (int64_t)wrow0 * ldw * ESZ, (uint32_t)((int64_t)nrows * ldw * ESZ));
    const uint32_t wlane = (uint32_t)((lane & 15) * ldw * ESZ + (int64_t)(k_begin + 4 * g) * ESZ);
    auto load_w = [&](int step, WReg& w) {
        if (VEC) {
            const uint32_t off = wlane + (uint32_t)(step * 32 * ESZ);
            if constexpr (WF16) {
                const auto a = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, off, 0, 0);
                const auto b = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, off + 16 * ESZ, 0, 0);
                w = WReg{a[0], a[1], b[0], b[1]};
            } else {
                const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off, 0, 0);
                const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(wrsrc, off + 16 * ESZ, 0, 0);
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

    floatx4 acc_hh[MT], acc_c[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) { acc_hh[t][e] = 0.f; acc_c[t][e] = 0.f; }

    // prologue: W for steps 0 .. PFW-1 and activation block 0 in flight
    // together; block 0 lands in LDS buffer 0 (split here, or copied, in
    // which case the copy is issued first so its wait leaves W in flight)
    WReg wr[PFW];
    if constexpr (INK) {
#pragma unroll
        for (int s = 0; s < PFW; ++s) load_w(min(s, nsteps - 1), wr[s]);
        load_a(0);
        __builtin_amdgcn_sched_barrier(0);
        store_a(0);
        __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    } else {
        dma_block(0);
#pragma unroll
        for (int s = 0; s < PFW; ++s) load_w(min(s, nsteps - 1), wr[s]);
        __builtin_amdgcn_sched_barrier(0);
        if (VEC) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PFW));   // block 0 landed; W still in flight
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();
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
        const unsigned char* abuf = sa + (b & 1) * BB;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
            const int step = b * STEPS + s;
            WReg& w = wr[J + s];
            half8 wh, wl;
            if constexpr (WF16) {
                wh = __builtin_bit_cast(half8, w);
            } else {
                const floatx8 wf = __builtin_bit_cast(floatx8, w);
                const float4 ra = {wf[0], wf[1], wf[2], wf[3]}, rb = {wf[4], wf[5], wf[6], wf[7]};
                split8(ra, rb, wh, wl);
                wmax = absmax8(wmax, ra, rb);
            }
            load_w(min(step + PFW, nsteps - 1), w);
            if (step < nsteps) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int off = ((s * MT + t) * 64 + lane) * 16;
                    const half8 ah = *reinterpret_cast<const half8*>(abuf + off);
                    const half8 al = *reinterpret_cast<const half8*>(abuf + BB / 2 + off);
                    mfma16(ah, wh, acc_hh[t]);
                    if constexpr (!WF16 && !ONE) mfma16(ah, wl, acc_c[t]);
                    if constexpr (!ONE) mfma16(al, wh, acc_c[t]);
                }
            }
        }
        if (more) {
            // the other buffer was last read in block b - 1, before the
            // previous barrier; it now holds (or receives) block b + 1
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (INK) {
                store_a(b + 1);
                __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
            } else {
                // the copy was issued before this block's 2 STEPS W loads
                if (VEC) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * STEPS));
                else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            __builtin_amdgcn_s_barrier();
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

    // ---- epilogue: lane holds column n, rows t*16 + 4g + e; each output is
    //      (acc_hh + 2^-10 acc_c) 2^-e_m --------------------------------------
    if (!row_ok) return;
    float* o = out + split * split_stride;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int4 er = *reinterpret_cast<const int4*>(aexp + t * 16 + 4 * g);
        const int ev[4] = {er.x, er.y, er.z, er.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = t * 16 + 4 * g + e;
            if (m < M) o[(int64_t)m * ldo + n] = __builtin_ldexpf(acc_hh[t][e] + acc_c[t][e] * 0.0009765625f, -ev[e]);
        }
    }
}

// C[m, n] = sum over chunks s (in order) of P[s, m, n].  The partials of a
// batch of chunks are loaded together (the clamped index keeps every load in
// bounds) and then added in chunk order, so the chain of adds waits on one
// round of loads per batch instead of one per chunk.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int splits,
                                                            int64_t M, int64_t N, float* __restrict__ C,
                                                            int64_t ldc) {
    constexpr int BATCH = 8;
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        float acc = 0.0f;
        for (int s0 = 0; s0 < splits; s0 += BATCH) {
            float v[BATCH];
#pragma unroll
            for (int j = 0; j < BATCH; ++j) v[j] = P[(int64_t)min(s0 + j, splits - 1) * total + i];
#pragma unroll
            for (int j = 0; j < BATCH; ++j)
                if (s0 + j < splits) acc = (s0 + j == 0) ? v[j] : acc + v[j];
        }
        const int64_t m = i / N, n = i - m * N;
        C[m * ldc + n] = acc;
    }
}

int mtiles(int64_t M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

}  // namespace

// workspace: row exponents (256 bytes), activation planes, split-K partials
constexpr int64_t kExpBytes = 256;
int64_t DecodePlan::bytes() const { return kExpBytes + (a_bytes + 255) / 256 * 256 + (p_bytes + 255) / 256 * 256; }

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
    p.a_bytes = mt == 1 ? 0 : ablocks * (mt == 2 ? block_bytes<2>() : block_bytes<4>());
    p.p_bytes = p.splits > 1 ? (p.splits * M * N * 4 + 255) / 256 * 256 : 0;
    return p;
}

hipError_t launch_gemm_decode(const float* A, int64_t lda, const int8_t* kshift, const void* W, bool wf16,
                              bool one, int64_t ldw, float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              void* workspace, const DecodePlan& plan, uint32_t* status, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    if (M > 64 || K == 0) return hipErrorInvalidValue;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    int* aexp = reinterpret_cast<int*>(ws);
    unsigned char* ablk = ws + kExpBytes;
    float* part = reinterpret_cast<float*>(ablk + (plan.a_bytes + 255) / 256 * 256);
    const int nablk = (int)((K + KA - 1) / KA);
    const int mt = mtiles(M);
    const int64_t nblk2 = (N + 2 * DEC_ROWS - 1) / (2 * DEC_ROWS);
    const bool wide = mt > 1 && nblk2 * plan.splits >= (mt == 4 ? WIDE_MIN_WG4 : WIDE_MIN_WG2);
    const int wg_rows = (wide ? 2 * NW : NW) * ROWS_PER_WAVE;
    const dim3 grid((unsigned)((N + wg_rows - 1) / wg_rows), (unsigned)plan.splits);
    float* out = plan.splits > 1 ? part : C;
    const int64_t ldo = plan.splits > 1 ? N : ldc;
    const int64_t stride = plan.splits > 1 ? M * N : 0;
    // W loads of 8 elements per step need rows aligned to the load width
    // (16 bytes fp32, 8 bytes fp16) and whole k32 steps
    const uintptr_t walign = wf16 ? 7 : 15;
    const bool vec = (reinterpret_cast<uintptr_t>(W) & walign) == 0 && (ldw & 3) == 0 && (K & 31) == 0;
    // activation units load as float4 when rows are 16-byte aligned
    const bool avec = (reinterpret_cast<uintptr_t>(A) & 15) == 0 && (lda & 3) == 0;
#define HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW_)                                      \
    hipLaunchKernelGGL((gemm_decode_kernel<MT_, VEC_, F16_, AV_, SH_, ONE_, NW_>), grid, dim3(64 * NW_), \
                       2 * block_bytes<MT_>(), s, A, lda, aexp, ablk, (int)plan.a_bytes, W, ldw, out, ldo, stride, \
                       (int)M, (int)N, (int)K, (int)plan.kchunk, kshift, status)
#define HEAL_DEC_LAUNCH(MT_, VEC_, F16_, AV_, SH_, ONE_)                                                \
    do {                                                                                                \
        if constexpr (MT_ > 1) {                                                                        \
            if (wide) HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, 2 * NW);                      \
            else HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW);                               \
        } else {                                                                                        \
            HEAL_DEC_LAUNCH_NW(MT_, VEC_, F16_, AV_, SH_, ONE_, NW);                                    \
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
        hipLaunchKernelGGL((decode_prep_kernel<MT_>), dim3(16 * (MT_)), dim3(256), 0, s, A, lda, (int)M,   \
                           (int)K, nablk, kshift, aexp, ablk);                                          \
        if (wf16) {                                                                                     \
            if (vec) HEAL_DEC_AV(MT_, true, true, SH_);                                                 \
            else HEAL_DEC_AV(MT_, false, true, SH_);                                                    \
        } else {                                                                                        \
            if (vec) HEAL_DEC_AV(MT_, true, false, SH_);                                                \
            else HEAL_DEC_AV(MT_, false, false, SH_);                                                   \
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
#undef HEAL_DEC_LAUNCH_NW
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const int64_t total = M * N;
    const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, plan.splits, M, N, C,
                       ldc);
    return hipGetLastError();
}

}  // namespace heal

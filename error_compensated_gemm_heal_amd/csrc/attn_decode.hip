// Decode attention over an INT16 KV cache, with the INT16 -> dual-FP16
// unpack fused into the operand load.
//
// HEAL paper, section 3, "Mitigating QKV Truncation Error via INT16
// Quantization": Q, K and V are stored as INT16 codes (one scale per token
// and head).  At compute time each code is unpacked into two FP16 values
// whose sum is the code, and attention is expanded into 16-bit products with
// FP32 accumulation.  The expansion needs more than three times the flops,
// but the kernel stays bound by HBM reads of the 16-bit cache.
//
// Unpack used here: a code q = 64 qh + ql with qh = q >> 6 (in [-512, 511])
// and ql = q & 63 (in [0, 63]); both are exact FP16 values.  The pages' form
// hi + lo' / 2^10 holds with hi = 64 qh and lo' = 1024 ql.  Both halves are
// made with packed 16-bit integer/fp16 operations (a shift or a mask, then
// an exponent bias and one packed subtract): 2.5 instructions per code.
// Every 16-bit product is exact in fp32.
//
// One block of 4 waves owns one (batch b, KV head g, range of 256 tokens);
// each wave takes 64 of them:
//  * all loads are issued first: K straight into MFMA operand registers
//    (lane = token, 8 consecutive d), V by direct-to-LDS loads into a
//    wave-private 16 KB tile whose 16-byte chunks are XOR-swizzled by row;
//  * scores as S^T = K . q^T on v_mfma_f32_16x16x32_f16.  The 16 rows are
//    tokens; the 16 columns pack [64 q_hi of the G heads | q_lo of the G
//    heads].  K_hi and K_lo have one accumulator each, and
//    k.q = 64 (S_hi[c] + S_hi[G+c]) + S_lo[c] + S_lo[G+c];
//  * softmax in base 2 (log2 e folded into the score scale s_q s_k / sqrt(D),
//    hardware exp2) against the maximum over the wave's 64 tokens, taken
//    before any product with V, so nothing is ever rescaled inside a wave;
//  * P.V: the token weight p_t s_v(t) 2^E (2^E a power of two per wave that
//    keeps the weights in [0, 2)) is split into fp16 hi/lo by round to
//    nearest.  The S^T register layout already is the MFMA A-operand layout
//    (lane = head, lane group = 4 + 4 tokens), so P needs no transpose.  The
//    rows pack [P_hi | P_lo].  The V operand (8 tokens of one d per lane) is
//    read from LDS with the transposing ds_read_b64_tr_b16; V_hi and V_lo
//    have one accumulator each;
//  * the 4 waves merge their (m, l, o) in LDS, each block writes one partial
//    for its range, and a second kernel merges the ranges of a head in
//    range order.
#include <algorithm>

#include "heal_internal.h"

namespace heal {

namespace {

constexpr int D = 128;
constexpr int TW = 64;                // tokens per wave
constexpr int WPB = 4;                // waves per block
constexpr int TB = TW * WPB;          // tokens per block
constexpr int VTILE = TW * D * 2;     // wave-private LDS bytes: V codes of 64 tokens
constexpr float kLog2eInvSqrtD = 0.12751743074602467f;   // log2(e) / sqrt(128)

typedef short short2v __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) short4v* lds_s4_ptr;

__device__ __forceinline__ void mfma16(const half8& a, const half8& b, floatx4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two int16 codes in one dword -> exact fp16 pairs (code >> 6) and (code & 63).
// code >> 6 lies in [-512, 511]: adding the fp16 pattern 0x6600 gives the
// fp16 number 1536 + (code >> 6) in [1024, 2047], where fp16 spacing is 1, and
// subtracting 1536 leaves it exactly.  code & 63 or'ed into 0x6400 is the fp16
// number 1024 + (code & 63).
__device__ __forceinline__ void unpack2(uint32_t w, half2v& hi, half2v& lo) {
    const short2v t = __builtin_bit_cast(short2v, w) >> (short2v)(short)6;
    const ushort2v u = __builtin_bit_cast(ushort2v, t) + (ushort2v)(unsigned short)0x6600;
    hi = __builtin_bit_cast(half2v, u) - (half2v)(_Float16)1536.0f;
    lo = __builtin_bit_cast(half2v, (w & 0x003F003Fu) | 0x64006400u) - (half2v)(_Float16)1024.0f;
}

// Same high halves; the low halves are left biased, as the fp16 numbers
// 1024 + (code & 63), in a single bit operation ((w & 0x003F003F) | 0x64006400).
// A product chain over biased low halves is started from -1024 times the sum
// of the other operand, which removes the bias: every product stays exact
// ((1024 + ql) has 11 significant bits), and the extra rounding is that of a
// partial sum at most 1087 / 64 times larger than the unbiased one, far below
// the rounding of the high-half chain it is added to.
__device__ __forceinline__ void unpack8_lobias(const u32x4& raw, half8& hi, half8& lob) {
    u32x4 hw, lw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = raw[i];
        const short2v t = __builtin_bit_cast(short2v, w) >> (short2v)(short)6;
        const ushort2v u = __builtin_bit_cast(ushort2v, t) + (ushort2v)(unsigned short)0x6600;
        hw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u) - (half2v)(_Float16)1536.0f);
        lw[i] = __builtin_amdgcn_bitop3_b32(w, 0x003F003Fu, 0x64006400u, 0xEA);   // (w & m) | b
    }
    hi = __builtin_bit_cast(half8, hw);
    lob = __builtin_bit_cast(half8, lw);
}

__device__ __forceinline__ void unpack8(const u32x4& raw, half8& hi, half8& lo) {
    u32x4 hw, lw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        half2v h, l;
        unpack2(raw[i], h, l);
        hw[i] = __builtin_bit_cast(uint32_t, h);
        lw[i] = __builtin_bit_cast(uint32_t, l);
    }
    hi = __builtin_bit_cast(half8, hw);
    lo = __builtin_bit_cast(half8, lw);
}

// Cross-lane steps without LDS instructions (VALU lane permutes and DPP), so
// that nothing before the wait for the direct-to-LDS V loads is an LDS access.
// v_permlane16_swap / v_permlane32_swap of x with itself hand each lane the
// value of lane ^ 16 / lane ^ 32 in one of the two results.
__device__ __forceinline__ float group_max(float x) {   // over lanes with equal lane % 16
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t w = __builtin_bit_cast(uint32_t, x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t w = __builtin_bit_cast(uint32_t, x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Lane c of each 16-lane row gets lane c + N (row_shl) or c - N (row_shr) of
// the same row; lanes whose source is outside the row get 0.
template <int N>
__device__ __forceinline__ float row_from_right(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + N, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float row_from_left(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}

// LDS placement of V: token row r of a wave tile holds its sixteen 16-byte
// chunks (8 d each) in slots chunk ^ vswz(r).  The transposing reads of P.V
// then touch 32 distinct 8-byte bank groups per 32 lanes.
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 7); }

template <int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const int16_t* __restrict__ q, const float* __restrict__ qs, const int16_t* __restrict__ k,
    const float* __restrict__ ks, const int16_t* __restrict__ v, const float* __restrict__ vs,
    float* __restrict__ part, int T, int Hkv, int units) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[WPB * VTILE];
    __shared__ float wm[WPB][8], wl[WPB][8], winv[WPB];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int ub = blockIdx.x % units;
    const int gk = (blockIdx.x / units) % Hkv;
    const int b = blockIdx.x / (units * Hkv);
    const int t_begin = ub * TB + wid * TW;
    // this wave's tokens (0 past the end); scalar, as the buffer resources are
    const int nt = __builtin_amdgcn_readfirstlane(max(0, min(TW, T - t_begin)));
    unsigned char* vt = lds + wid * VTILE;

    const int c = lane & 15, grp = lane >> 4;
    const int Hq = G * Hkv;
    const int64_t tok_stride = (int64_t)Hkv * D;                  // int16 elements between tokens
    const uint32_t row_bytes = (uint32_t)(tok_stride * 2);

    // K and V of this wave's tokens through buffer resources that end at its
    // last token (so no read reaches another wave's tokens or past the
    // cache: those return zeros).  All offsets are per lane.
    const int tfirst = __builtin_amdgcn_readfirstlane(min(t_begin, T - 1));
    const int64_t tok0 = ((int64_t)b * T + tfirst) * Hkv + gk;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + tok0 * D, (uint32_t)nt * row_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + tok0 * D, (uint32_t)nt * row_bytes);

    // ---- loads, in the order they are needed: q and the token scales, K,
    //      then V.  They are unconditional, from clamped in-range indices
    //      (unused values are dropped afterwards), so no branch splits them.
    const int head = c < G ? c : (c < 2 * G ? c - G : 0);
    const int16_t* qrow = q + ((int64_t)b * Hq + gk * G + head) * D;
    u32x4 qraw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * grp);
    const float qscale_raw = qs[(int64_t)b * Hq + gk * G + head];
    // token scales where the score and weight layouts need them: ksv[4 st + e]
    // and vsv[4 st + e] belong to token 16 st + 4 grp + e (0 past the wave's
    // tokens, by the resource bound)
    float ksv[16], vsv[16];
    {
        const uint32_t srec = nt > 0 ? (uint32_t)(((nt - 1) * Hkv + 1) * 4) : 0u;
        const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(ks + tok0, srec);
        const __amdgpu_buffer_rsrc_t vsrs = make_rsrc(vs + tok0, srec);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t off = (uint32_t)((16 * (i >> 2) + 4 * grp + (i & 3)) * Hkv * 4);
            ksv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksrs, off, 0, 0));
            vsv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsrs, off, 0, 0));
        }
    }

    // K: lane (c, grp) of score block st gets token 16 st + c,
    // d = 32 s + 8 grp + j (j < 8), in kr[4 st + s]
    u32x4 kr[16];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            kr[4 * st + s] = __builtin_amdgcn_raw_buffer_load_b128(
                krs, (uint32_t)(16 * st + c) * row_bytes + (uint32_t)(64 * s + 16 * grp), 0, 0);
    // V into LDS: load i fills rows 4 i .. 4 i + 3; lane L writes row
    // 4 i + L / 16, slot L % 16, which holds chunk slot ^ vswz(row)
    {
        const int r_in = lane >> 4;
        const uint32_t v_even = (uint32_t)r_in * row_bytes + 16u * (uint32_t)((lane & 15) ^ vswz(r_in));
        const uint32_t v_odd = (uint32_t)r_in * row_bytes + 16u * (uint32_t)((lane & 15) ^ vswz(4 + r_in));
#pragma unroll
        for (int i = 0; i < TW / 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr)(vt + 1024 * i), 16,
                                                     ((i & 1) ? v_odd : v_even) + (uint32_t)(4 * i) * row_bytes,
                                                     0, 0, 0);
    }

    // ---- q as the packed B operand: column c < G -> 64 (q >> 6) of head c,
    //      G <= c < 2G -> q & 63 of head c - G, else 0.  d = 32 s + 8 grp + j.
    // (selected by exact fp16 factors 64 / 1 / 0 rather than by branches)
    half8 qf[4];
    {
        const _Float16 fh = c < G ? (_Float16)64.0f : (_Float16)0.0f;
        const _Float16 fl = (c >= G && c < 2 * G) ? (_Float16)1.0f : (_Float16)0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 hi, lo;
            unpack8(qraw[s], hi, lo);
            qf[s] = hi * fh + lo * fl;
        }
    }
    const float qscale = c < G ? qscale_raw : 0.0f;
    // power of two keeping s_v(t) 2^E in [1, 2) for this wave's tokens (the
    // four rows of lanes together hold all 64 of them)
    float vmax = vsv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) vmax = fmaxf(vmax, vsv[i]);
    vmax = group_max(vmax);
    int vexp = 0;
    (void)frexpf(vmax, &vexp);                                  // vmax in [2^(vexp-1), 2^vexp)
    const float p2 = vmax > 0.0f ? ldexpf(1.0f, 1 - vexp) : 1.0f;

    // ---- scores for 4 x 16 tokens; sc[4 st + e] is token 16 st + 4 grp + e.
    //      The K low halves come biased by 1024; their chains start from
    //      qbias[col] = -1024 * sum_d q_col[d] (an MFMA against a constant
    //      -1024 row, exact: integer sums below 2^24).
    floatx4 qbias = {0.f, 0.f, 0.f, 0.f};
    {
        const half8 m1024 = (half8)(_Float16)-1024.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) mfma16(m1024, qf[s], qbias);
    }
    float sc[16];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        floatx4 s_hi = {0.f, 0.f, 0.f, 0.f}, s_lo = qbias;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 kh, kl;
            unpack8_lobias(kr[4 * st + s], kh, kl);
            mfma16(kh, qf[s], s_hi);
            mfma16(kl, qf[s], s_lo);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float part_c = 64.0f * s_hi[e] + s_lo[e];
            const float dot = part_c + row_from_right<G>(part_c);      // + the q & 63 column
            const int tl = 16 * st + 4 * grp + e;
            // masked by adding -inf (the product is finite), so the scale
            // load is consumed unconditionally and stays with the others
            const float mask = (c < G && tl < nt) ? 0.0f : -INFINITY;
            sc[4 * st + e] = dot * (qscale * ksv[4 * st + e] * kLog2eInvSqrtD) + mask;
        }
    }
    float m = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, sc[i]);
    m = group_max(m);
    const bool live = m > -INFINITY;                   // a head lane with at least one token
    float p[16], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        p[i] = live ? __builtin_amdgcn_exp2f(sc[i] - m) : 0.0f;
        psum += p[i];
    }
    const float l = group_sum(psum);

    // ---- P.V operand A for token blocks kb = 0, 1 (32 tokens each): row
    //      c < G -> fp16 hi of head c's weight, G <= c < 2G -> fp16 lo of head
    //      c - G's weight.  Slot i = token 32 kb + 16 (i / 4) + 4 grp + i % 4.
    half8 pa[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float w = p[8 * kb + i] * vsv[8 * kb + i] * p2;
            const float wo = row_from_left<G>(w);
            _Float16 h, lo;
            split_one(c < G ? w : wo, h, lo);
            pa[kb][i] = c < G ? h : (c < 2 * G ? lo : (_Float16)0.0f);
        }

    // ---- V operand by transposing LDS reads.  In each 16-lane group, lane
    //      4 j + x supplies the address of 4 d starting at 16 dt + 4 x of token
    //      row 4 grp + j (+ 16 h + 32 kb); lane i then receives d = 16 dt + i of
    //      those 4 tokens, which are slots 4 h .. 4 h + 3.
    __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): V is in LDS
    __builtin_amdgcn_sched_barrier(0);
    // V low halves come biased by 1024: their chains start from
    // pbias[row] = -1024 * sum_t P[row][t] (an MFMA against a constant
    // -1024 column block), the same for every d.
    floatx4 pbias = {0.f, 0.f, 0.f, 0.f};
    {
        const half8 m1024 = (half8)(_Float16)-1024.0f;
        mfma16(pa[0], m1024, pbias);
        mfma16(pa[1], m1024, pbias);
    }
    floatx4 acc_h[8], acc_l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc_l[i] = pbias;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc_h[i][e] = 0.0f;
    }
    {
        const int s16 = lane & 15;
        const int rr = 4 * grp + (s16 >> 2);           // row within a 16-row half, mod 8 = vswz input
        const int lane_off = rr * (D * 2) + 16 * ((s16 & 3) >> 1) + 8 * (s16 & 1);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int off = lane_off + 16 * ((2 * dt) ^ vswz(rr));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const short4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s4_ptr)(vt + off + (32 * kb) * (D * 2)));
                const short4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s4_ptr)(vt + off + (32 * kb + 16) * (D * 2)));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo4), hi2 = __builtin_bit_cast(u32x2, hi4);
                const u32x4 raw = {lo2.x, lo2.y, hi2.x, hi2.y};
                half8 vh, vl;
                unpack8_lobias(raw, vh, vl);
                mfma16(pa[kb], vh, acc_h[dt]);
                mfma16(pa[kb], vl, acc_l[dt]);
            }
        }
    }

    // ---- stage this wave's rows R = 64 acc_h + acc_l (2G rows of D) in its
    //      own LDS tile (after its own reads), plus (m, l, 1 / 2^E)
    float* ob = reinterpret_cast<float*>(vt);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * grp + e;
            if (r < 2 * G) ob[r * D + 16 * dt + c] = 64.0f * acc_h[dt][e] + acc_l[dt][e];
        }
    if (lane < G) {
        wm[wid][lane] = m;
        wl[wid][lane] = l;
    }
    if (lane == 0) winv[wid] = 1.0f / p2;
    __syncthreads();

    // ---- merge the 4 waves: o[h][d] = (R[h][d] + R[G+h][d] / 2^10) / 2^E
    float* pout = part + (int64_t)blockIdx.x * (2 * G + G * D);
    for (int i = threadIdx.x; i < G * D; i += 256) {
        const int h = i / D, d = i - h * D;
        float M = wm[0][h];
#pragma unroll
        for (int w = 1; w < WPB; ++w) M = fmaxf(M, wm[w][h]);
        float O = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < WPB; ++w) {
            const float mw = wm[w][h];
            const float f = mw > -INFINITY ? __builtin_amdgcn_exp2f(mw - M) : 0.0f;
            const float* R = reinterpret_cast<const float*>(lds + w * VTILE);
            O += f * ((R[h * D + d] + R[(G + h) * D + d] * 0.0009765625f) * winv[w]);
            L += f * wl[w][h];
        }
        pout[2 * G + i] = O;
        if (d == 0) {
            pout[h] = M;
            pout[G + h] = L;
        }
    }
}

// Merge the token ranges of one (b, h), in range order:
//   out = sum_u w_u o_u / sum_u w_u l_u,   w_u = 2^(m_u - max_u m_u).
// Up to four groups of D threads (one d each; one group per 8 ranges) take
// consecutive shares of the ranges; each folds (m_u, l_u, o_u[d]) of its share
// into a running (M, L, O), loading CB ranges at a time with independent
// loads, and group 0 merges the groups in order.  The order depends on the
// number of ranges only.
constexpr int CNG = 4;   // most range groups per (b, h)
constexpr int CB = 8;    // ranges per round of loads
int combine_groups(int units) { return std::min(CNG, (units + CB - 1) / CB); }
__global__ __launch_bounds__(CNG * D) void attn_combine_kernel(const float* __restrict__ part,
                                                               float* __restrict__ out, int Hq, int Hkv,
                                                               int G, int units) {
    __shared__ float sm[CNG], sl[CNG], so[CNG][D];
    const int bh = blockIdx.x;
    const int b = bh / Hq, h = bh - b * Hq;
    const int gk = h / G, c = h - gk * G;
    const int d = threadIdx.x % D;
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / D);
    const int ng = blockDim.x / D;
    const int per = (units + ng - 1) / ng;
    const int ub = grp * per, ue = min(units, ub + per);
    const int64_t stride = 2 * G + G * D;
    const float* base = part + ((int64_t)b * Hkv + gk) * units * stride;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int u0 = ub; u0 < ue; u0 += CB) {
        float mu[CB], lu[CB], ou[CB];
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const int u = min(u0 + i, ue - 1);
            mu[i] = base[u * stride + c];
            lu[i] = base[u * stride + G + c];
            ou[i] = base[u * stride + 2 * G + c * D + d];
        }
        float mc = M;
#pragma unroll
        for (int i = 0; i < CB; ++i)
            if (u0 + i < ue) mc = fmaxf(mc, mu[i]);
        const float r = M > -INFINITY ? __builtin_amdgcn_exp2f(M - mc) : 0.0f;
        L *= r;
        O *= r;
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            const float w = (u0 + i < ue && mu[i] > -INFINITY) ? __builtin_amdgcn_exp2f(mu[i] - mc) : 0.0f;
            L += w * lu[i];
            O += w * ou[i];
        }
        M = mc;
    }
    if (d == 0) {
        sm[grp] = M;
        sl[grp] = L;
    }
    so[grp][d] = O;
    __syncthreads();
    if (grp == 0) {
        // every range holds at least one token with a finite score, so the
        // maximum over the groups is finite; an empty group carries weight 0
        float mx = sm[0];
        for (int g = 1; g < ng; ++g) mx = fmaxf(mx, sm[g]);
        float Lt = 0.0f, Ot = 0.0f;
        for (int g = 0; g < ng; ++g) {
            const float w = sm[g] > -INFINITY ? __builtin_amdgcn_exp2f(sm[g] - mx) : 0.0f;
            Lt += w * sl[g];
            Ot += w * so[g][d];
        }
        out[(int64_t)bh * D + d] = Ot / Lt;
    }
}

}  // namespace

int64_t attn_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dd) {
    (void)Dd;
    const int64_t G = Hq / Hkv;
    const int64_t units = (T + TB - 1) / TB;
    return (B * Hkv * units * (2 * G + G * D) * 4 + 255) / 256 * 256;
}

hipError_t launch_attn_decode(const int16_t* q, const float* qs, const int16_t* k, const float* ks,
                              const int16_t* v, const float* vs, float* out, int64_t B, int64_t T,
                              int64_t Hq, int64_t Hkv, int64_t Dd, void* workspace, hipStream_t s) {
    if (Dd != D) return hipErrorInvalidValue;
    const int G = (int)(Hq / Hkv);
    const int units = (int)((T + TB - 1) / TB);
    const unsigned blocks = (unsigned)(B * Hkv * units);
    float* part = static_cast<float*>(workspace);
#define HEAL_ATT(G_)                                                                                \
    case G_:                                                                                        \
        hipLaunchKernelGGL((attn_decode_kernel<G_>), dim3(blocks), dim3(256), 0, s, q, qs, k, ks, v, \
                           vs, part, (int)T, (int)Hkv, units);                              \
        break;
    switch (G) {
        HEAL_ATT(1) HEAL_ATT(2) HEAL_ATT(3) HEAL_ATT(4) HEAL_ATT(5) HEAL_ATT(6) HEAL_ATT(7) HEAL_ATT(8)
        default: return hipErrorInvalidValue;
    }
#undef HEAL_ATT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(B * Hq)), dim3(combine_groups(units) * D), 0, s, part, out, (int)Hq,
                       (int)Hkv, G, units);
    return hipGetLastError();
}

}  // namespace heal

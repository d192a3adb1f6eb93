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
// One wave owns one (batch b, KV head g, range of TW tokens):
//  * scores as S^T = K . q^T on v_mfma_f32_16x16x32_f16.  The 16 rows are
//    tokens; K goes from HBM straight into operand registers (lane = token,
//    8 consecutive d), then is unpacked.  The 16 columns pack
//    [64 q_hi of the G heads | q_lo of the G heads].  K_hi and K_lo have one
//    accumulator each, and k.q = 64 (S_hi[c] + S_hi[G+c]) + S_lo[c] + S_lo[G+c];
//  * fp32 online softmax per head in base 2 (log2 e folded into the score
//    scale s_q s_k / sqrt(D), hardware exp2), rescaling the running output
//    only when a head's maximum rises by more than 2^8;
//  * P.V: the token weight p_t s_v(t) 2^E (2^E a power of two per wave that
//    keeps the weights in fp16 range) is split into fp16 hi/lo by round to
//    nearest.  The S^T register layout already is the MFMA A-operand layout
//    (lane = head, lane group = 4 + 4 tokens), so no transpose of P is
//    needed.  The rows pack [P_hi | P_lo].  V codes go through a
//    wave-private LDS tile (the operand needs 8 tokens of one d per lane),
//    with one accumulator for V_hi and one for V_lo;
//  * the wave's token scales are loaded once and handed to the lanes that
//    need them with lane shuffles;
//  * each wave writes (m, l, o) for its range, and a second kernel merges
//    the ranges of a head in range order.
#include "heal_internal.h"

namespace heal {

namespace {

constexpr int D = 128;
constexpr int TW = 128;               // tokens per wave
constexpr int VROW = D * 2 + 16;      // LDS bytes per V token row (padded)
constexpr int VTILE = 32 * VROW;      // wave-private LDS bytes
constexpr float kLog2eInvSqrtD = 0.12751743074602467f;   // log2(e) / sqrt(128)

typedef short short2v __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ float group_max(float x) {   // over lanes with equal lane % 16
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float group_sum(float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

template <int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(
    const int16_t* __restrict__ q, const float* __restrict__ qs, const int16_t* __restrict__ k,
    const float* __restrict__ ks, const int16_t* __restrict__ v, const float* __restrict__ vs,
    float* __restrict__ part, int B, int T, int Hkv, int units) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[4 * VTILE];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t gw = (int64_t)blockIdx.x * 4 + wid;
    if (gw >= (int64_t)B * Hkv * units) return;
    const int u = (int)(gw % units);
    const int gk = (int)((gw / units) % Hkv);
    const int b = (int)(gw / ((int64_t)units * Hkv));
    const int t_begin = u * TW, t_end = min(T, t_begin + TW);
    unsigned char* vt = lds + wid * VTILE;

    const int c = lane & 15, grp = lane >> 4;
    const int Hq = G * Hkv;
    const int64_t tok_stride = (int64_t)Hkv * D;               // int16 elements between tokens
    // K and V of (b, gk) are read through buffer resources that start at the
    // current tile and end at token T: a read past the cache returns zeros,
    // so loads need no per-lane guards (tokens outside this wave's range are
    // masked through their scores and weights instead).  The resources are
    // scalar; lane offsets stay below 32 token rows.
    const uint32_t row_bytes = (uint32_t)(tok_stride * 2);
    const uint32_t region = (uint32_t)T * row_bytes;             // < 2^32, checked by the caller
    const int16_t* kb = k + ((int64_t)b * T * Hkv + gk) * D;
    const int16_t* vb = v + ((int64_t)b * T * Hkv + gk) * D;
    const float* ksb = ks + (int64_t)b * T * Hkv + gk;
    const float* vsb = vs + (int64_t)b * T * Hkv + gk;

    // ---- q as the packed B operand: column c < G -> 64 (q >> 6) of head c,
    //      G <= c < 2G -> q & 63 of head c - G, else 0.  d = 32 s + 8 grp + j.
    half8 qf[4];
    {
        const int head = c < G ? c : c - G;
        const bool use = c < 2 * G;
        const int16_t* qrow = q + ((int64_t)b * Hq + gk * G + (use ? head : 0)) * D;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 raw = use ? *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * grp) : (u32x4)(0u);
            half8 hi, lo;
            unpack8(raw, hi, lo);
            qf[s] = c < G ? hi * (_Float16)64.0f : lo;
        }
    }
    const float qscale = c < G ? qs[(int64_t)b * Hq + gk * G + c] : 0.0f;

    // ---- this wave's token scales: lane l holds tokens t_begin + l and + 64 + l
    const float ks0 = (t_begin + lane < t_end) ? ksb[(int64_t)(t_begin + lane) * Hkv] : 0.0f;
    const float ks1 = (t_begin + 64 + lane < t_end) ? ksb[(int64_t)(t_begin + 64 + lane) * Hkv] : 0.0f;
    const float vs0 = (t_begin + lane < t_end) ? vsb[(int64_t)(t_begin + lane) * Hkv] : 0.0f;
    const float vs1 = (t_begin + 64 + lane < t_end) ? vsb[(int64_t)(t_begin + 64 + lane) * Hkv] : 0.0f;

    // ---- power of two keeping s_v(t) 2^E in [1, 2) for this wave's tokens ----
    float vmax = fmaxf(vs0, vs1);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    int vexp = 0;
    (void)frexpf(vmax, &vexp);                                  // vmax in [2^(vexp-1), 2^vexp)
    const float p2 = vmax > 0.0f ? ldexpf(1.0f, 1 - vexp) : 1.0f;

    float m_run = -INFINITY, l_run = 0.0f;
    floatx4 acc_h[8], acc_l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) { acc_h[i][e] = 0.0f; acc_l[i][e] = 0.0f; }

    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        const int t0l = t0 - t_begin;                // 0, 32, 64 or 96: uniform
        const float ksel = t0l < 64 ? ks0 : ks1;
        const float vsel = t0l < 64 ? vs0 : vs1;
        // ---- V tile -> wave-private LDS (issued first, consumed last) -------
        const uint32_t tile_off = (uint32_t)t0 * row_bytes;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kb + (int64_t)t0 * tok_stride, region - tile_off);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vb + (int64_t)t0 * tok_stride, region - tile_off);
        u32x4 vraw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {                 // 32 rows x 16 chunks of 16 bytes
            const int chunk = lane + 64 * i;
            vraw[i] = __builtin_amdgcn_raw_buffer_load_b128(
                vrs, (uint32_t)(chunk >> 4) * row_bytes + (uint32_t)(chunk & 15) * 16u, 0, 0);
        }
        // ---- scores S^T for 2 x 16 tokens ------------------------------------
        float sc[8];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            u32x4 kr[4];
            const uint32_t koff = (uint32_t)(16 * st + c) * row_bytes + (uint32_t)grp * 16u;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kr[s] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 64u * s, 0, 0);
            floatx4 s_hi = {0.f, 0.f, 0.f, 0.f}, s_lo = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8 kh, kl;
                unpack8(kr[s], kh, kl);
                mfma16(kh, qf[s], s_hi);
                mfma16(kl, qf[s], s_lo);
            }
            // lane (c, grp), reg e: token t0 + 16 st + 4 grp + e, column c
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float part_c = 64.0f * s_hi[e] + s_lo[e];
                const float dot = part_c + __shfl_down(part_c, G, 16);     // + the q & 63 column
                const int tl = t0l + 16 * st + 4 * grp + e;               // token within the wave
                const float kscale = __shfl(ksel, tl & 63, 64);
                const bool valid = c < G && t0 + 16 * st + 4 * grp + e < t_end;
                sc[4 * st + e] = valid ? dot * (qscale * kscale * kLog2eInvSqrtD) : -INFINITY;
            }
        }
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
        mt = group_max(mt);
        // Lazy rescale: the reference maximum of a head moves only when the
        // scores pass it by more than 8 (log2 units), so unscaled weights stay
        // below 2^8 (fp16-safe after the scale fold) and the running output
        // is rescaled on rare tiles only.
        const bool bump = c < G && mt > m_run + 8.0f;   // always true on the first tile
        if (__builtin_amdgcn_ballot_w64(bump)) {
            const float m_new = bump ? mt : m_run;
            const float alpha = c < G ? (m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new)) : 0.0f;
            l_run *= alpha;
            m_run = m_new;
#pragma unroll
            for (int e = 0; e < 4; ++e) {   // rows of the running output, by head
                const int r = 4 * grp + e;
                const int hr = r < G ? r : (r < 2 * G ? r - G : 0);
                const float ar = __shfl(alpha, hr, 64);
                const float f = r < 2 * G ? ar : 0.0f;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    acc_h[dt][e] *= f;
                    acc_l[dt][e] *= f;
                }
            }
        }
        float p[8], psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = c < G ? __builtin_amdgcn_exp2f(sc[i] - m_run) : 0.0f;
            psum += p[i];
        }
        l_run += group_sum(psum);

        // ---- P.V operand A: row c < G -> fp16 hi of head c's weight, row
        //      G <= c < 2G -> fp16 lo of head c - G's weight.  Slot i = token
        //      t0 + 16 (i / 4) + 4 grp + i % 4, the same slots V uses below.
        half8 pa;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tl = t0l + 16 * (i >> 2) + 4 * grp + (i & 3);
            const float vscale = __shfl(vsel, tl & 63, 64);
            const float w = p[i] * vscale * p2;
            const float wo = __shfl_up(w, G, 16);
            _Float16 h, l;
            split_one(c < G ? w : wo, h, l);
            pa[i] = c < G ? h : (c < 2 * G ? l : (_Float16)0.0f);
        }
        // ---- V tile into LDS, then 8 d-tiles of 16 ---------------------------
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int chunk = lane + 64 * i;
            *reinterpret_cast<u32x4*>(vt + (chunk >> 4) * VROW + (chunk & 15) * 16) = vraw[i];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int d = 16 * dt + c;
            u32x4 raw;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i0 = 2 * jj, i1 = 2 * jj + 1;
                const int r0 = 16 * (i0 >> 2) + 4 * grp + (i0 & 3);
                const int r1 = 16 * (i1 >> 2) + 4 * grp + (i1 & 3);
                const uint16_t a0 = *reinterpret_cast<const uint16_t*>(vt + r0 * VROW + 2 * d);
                const uint16_t a1 = *reinterpret_cast<const uint16_t*>(vt + r1 * VROW + 2 * d);
                raw[jj] = (uint32_t)a0 | ((uint32_t)a1 << 16);
            }
            half8 vh, vl;
            unpack8(raw, vh, vl);
            mfma16(pa, vh, acc_h[dt]);
            mfma16(pa, vl, acc_l[dt]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- write this range's (m, l, o): row r = 64 acc_h + acc_l;
    //      o[h][d] = row h + row (G + h) / 2^10, divided by the power of two
    //      folded into the weights.  m is in base 2.
    float* ob = reinterpret_cast<float*>(vt);        // [2G][D] staging, reuses the V tile
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * grp + e;
            if (r < 2 * G) ob[r * D + 16 * dt + c] = 64.0f * acc_h[dt][e] + acc_l[dt][e];
        }
    __builtin_amdgcn_wave_barrier();
    float* pout = part + gw * (int64_t)(2 * G + G * D);
    if (lane < G) {
        pout[lane] = m_run;
        pout[G + lane] = l_run;
    }
    const float inv_p2 = 1.0f / p2;
    for (int i = lane; i < G * D; i += 64) {
        const int h = i / D, d = i - h * D;
        pout[2 * G + i] = (ob[h * D + d] + ob[(G + h) * D + d] * 0.0009765625f) * inv_p2;
    }
}

// Merge the token ranges of one (b, h), in range order:
//   out = sum_u w_u o_u / sum_u w_u l_u,   w_u = 2^(m_u - max_u m_u).
// The per-range weights are computed once into LDS; every thread then sums its
// d over the ranges with independent loads.
constexpr int kMaxUnits = 2048;
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part,
                                                           float* __restrict__ out, int Hq, int Hkv,
                                                           int G, int units) {
    __shared__ float wsh[kMaxUnits];
    __shared__ float red[4];
    const int bh = blockIdx.x;
    const int b = bh / Hq, h = bh - b * Hq;
    const int gk = h / G, c = h - gk * G;
    const int d = threadIdx.x;
    const int64_t stride = 2 * G + G * D;
    const float* base = part + ((int64_t)b * Hkv + gk) * units * stride;
    // maximum over ranges (two waves)
    float mloc = -INFINITY;
    for (int u = d; u < units; u += blockDim.x) mloc = fmaxf(mloc, base[u * stride + c]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off, 64));
    if ((d & 63) == 0) red[d >> 6] = mloc;
    __syncthreads();
    const float M = fmaxf(red[0], red[1]);
    float lloc = 0.0f;
    for (int u = d; u < units; u += blockDim.x) {
        const float w = __builtin_amdgcn_exp2f(base[u * stride + c] - M);
        wsh[u] = w;
        lloc += w * base[u * stride + G + c];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lloc += __shfl_xor(lloc, off, 64);
    if ((d & 63) == 0) red[2 + (d >> 6)] = lloc;
    __syncthreads();
    const float L = red[2] + red[3];
    float O = 0.0f;
#pragma unroll 8
    for (int u = 0; u < units; ++u) O += wsh[u] * base[u * stride + 2 * G + c * D + d];
    out[(int64_t)bh * D + d] = O / L;
}

}  // namespace

int64_t attn_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dd) {
    (void)Dd;
    const int64_t G = Hq / Hkv;
    const int64_t units = (T + TW - 1) / TW;
    return (B * Hkv * units * (2 * G + G * D) * 4 + 255) / 256 * 256;
}

hipError_t launch_attn_decode(const int16_t* q, const float* qs, const int16_t* k, const float* ks,
                              const int16_t* v, const float* vs, float* out, int64_t B, int64_t T,
                              int64_t Hq, int64_t Hkv, int64_t Dd, void* workspace, hipStream_t s) {
    if (Dd != D) return hipErrorInvalidValue;
    const int G = (int)(Hq / Hkv);
    const int units = (int)((T + TW - 1) / TW);
    if (units > kMaxUnits) return hipErrorInvalidValue;   // T up to 262144 tokens
    const int64_t waves = B * Hkv * units;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    float* part = static_cast<float*>(workspace);
#define HEAL_ATT(G_)                                                                                \
    case G_:                                                                                        \
        hipLaunchKernelGGL((attn_decode_kernel<G_>), dim3(blocks), dim3(256), 0, s, q, qs, k, ks, v, \
                           vs, part, (int)B, (int)T, (int)Hkv, units);                              \
        break;
    switch (G) {
        HEAL_ATT(1) HEAL_ATT(2) HEAL_ATT(3) HEAL_ATT(4) HEAL_ATT(5) HEAL_ATT(6) HEAL_ATT(7) HEAL_ATT(8)
        default: return hipErrorInvalidValue;
    }
#undef HEAL_ATT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(B * Hq)), dim3(D), 0, s, part, out, (int)Hq,
                       (int)Hkv, G, units);
    return hipGetLastError();
}

}  // namespace heal

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
// Unpack used here: hi = q - (q mod 64) (a multiple of 64, at most 10
// significant bits) and lo = q mod 64.  Both are exact FP16 values, and
// hi + lo == q exactly.  The pages' form hi + lo' / 2^10 holds with
// lo' = 1024 lo.  The products hi.hi, hi.lo, lo.hi and lo.lo are all exact
// in fp32.
//
// One wave owns one (batch b, KV head g, range of TW tokens):
//  * scores as S^T = K . q^T on v_mfma_f32_16x16x32_f16.  The 16 rows are
//    tokens; K goes from HBM straight into operand registers (lane = token,
//    8 consecutive d), then is unpacked.  The 16 columns pack
//    [q_hi of the G heads | q_lo of the G heads], so K_hi and K_lo each take
//    one MFMA per 32 d, both into the same accumulator.  The two column
//    halves are added across lanes afterwards;
//  * fp32 online softmax per head.  The scale s_q s_k / sqrt(D) is applied
//    in fp32;
//  * P.V: the token weight p_t s_v(t) 2^E (2^E a power of two per wave that
//    keeps the weights in fp16 range) is split into fp16 hi/lo by round to
//    nearest.  The S^T register layout already is the MFMA A-operand layout
//    (lane = head, lane group = 4 + 4 tokens), so no transpose of P is
//    needed.  The rows pack [P_hi | P_lo].  V codes go through a
//    wave-private LDS tile, since the operand needs 8 tokens of one d per
//    lane, and are unpacked as above;
//  * each wave writes (m, l, o) for its range, and a second kernel merges
//    the ranges of a head in range order.
#include "heal_internal.h"

namespace heal {

namespace {

constexpr int D = 128;
constexpr int TW = 128;               // tokens per wave
constexpr int VROW = D * 2 + 16;      // LDS bytes per V token row (padded)
constexpr int VTILE = 32 * VROW;      // wave-private LDS bytes
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

__device__ __forceinline__ void mfma16(const half8& a, const half8& b, floatx4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 int16 codes -> exact fp16 parts hi = q - (q & 63), lo = q & 63.
__device__ __forceinline__ void unpack8(const uint4& raw, half8& hi, half8& lo) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const short a = (short)(w[i] & 0xffffu), b = (short)(w[i] >> 16);
        hi[2 * i] = (_Float16)(short)(a & ~63);
        hi[2 * i + 1] = (_Float16)(short)(b & ~63);
        lo[2 * i] = (_Float16)(short)(a & 63);
        lo[2 * i + 1] = (_Float16)(short)(b & 63);
    }
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
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
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
    const int16_t* kbase = k + ((int64_t)b * T * Hkv + gk) * D;
    const int16_t* vbase = v + ((int64_t)b * T * Hkv + gk) * D;
    const float* ksb = ks + (int64_t)b * T * Hkv + gk;
    const float* vsb = vs + (int64_t)b * T * Hkv + gk;

    // ---- q as the packed B operand: column c < G -> hi part of head c,
    //      G <= c < 2G -> lo part of head c - G, else 0.  d = 32 s + 8 grp + j.
    half8 qf[4];
    {
        const int head = c < G ? c : c - G;
        const bool use = c < 2 * G;
        const int16_t* qrow = q + ((int64_t)b * Hq + gk * G + (use ? head : 0)) * D;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 raw = use ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * grp) : make_uint4(0, 0, 0, 0);
            half8 hi, lo;
            unpack8(raw, hi, lo);
            qf[s] = c < G ? hi : lo;
        }
    }
    const float qscale = c < G ? qs[(int64_t)b * Hq + gk * G + c] : 0.0f;

    // ---- power of two keeping s_v(t) 2^E in [1, 2) for this wave's tokens ----
    float vmax = 0.0f;
    for (int t = t_begin + lane; t < t_end; t += 64) vmax = fmaxf(vmax, vsb[(int64_t)t * Hkv]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    int vexp = 0;
    (void)frexpf(vmax, &vexp);                                  // vmax in [2^(vexp-1), 2^vexp)
    const float p2 = vmax > 0.0f ? ldexpf(1.0f, 1 - vexp) : 1.0f;

    float m_run = -INFINITY, l_run = 0.0f;
    floatx4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = 0.0f;

    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        // ---- V tile -> wave-private LDS (issued first, consumed last) -------
        uint4 vraw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int chunk = lane + 64 * i;          // 32 rows x 16 chunks of 16 bytes
            const int row = chunk >> 4, piece = chunk & 15;
            const int tok = t0 + row;
            vraw[i] = tok < t_end ? *reinterpret_cast<const uint4*>(vbase + tok * tok_stride + 8 * piece)
                                  : make_uint4(0, 0, 0, 0);
        }
        // ---- scores S^T for 2 x 16 tokens ------------------------------------
        floatx4 S[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int tok = t0 + 16 * st + c;
            const bool ok = tok < t_end;
            uint4 kr[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kr[s] = ok ? *reinterpret_cast<const uint4*>(kbase + tok * tok_stride + 32 * s + 8 * grp)
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[st][e] = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8 kh, kl;
                unpack8(kr[s], kh, kl);
                mfma16(kh, qf[s], S[st]);
                mfma16(kl, qf[s], S[st]);
            }
        }
        // lane (c, grp), reg e of S[st]: token t0 + 16 st + 4 grp + e, column c
        float sc[8];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float other = __shfl_down(S[st][e], G, 16);   // the q_lo column of this head
                const int tok = t0 + 16 * st + 4 * grp + e;
                const float kscale = tok < t_end ? ksb[(int64_t)tok * Hkv] : 0.0f;
                const float dot = S[st][e] + other;
                sc[4 * st + e] = (c < G && tok < t_end) ? dot * (qscale * kscale * kInvSqrtD) : -INFINITY;
            }
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
        mt = group_max(mt);
        const float m_new = fmaxf(m_run, mt);
        // lanes c >= G carry no head: keep their weights at zero
        const float alpha = (c < G && m_run != -INFINITY) ? expf(m_run - m_new) : 0.0f;
        float p[8], psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = c < G ? expf(sc[i] - m_new) : 0.0f;
            psum += p[i];
        }
        psum = group_sum(psum);
        l_run = l_run * alpha + psum;
        m_run = (c < G) ? m_new : -INFINITY;

        // ---- P.V operand A: row c < G -> fp16 hi of head c's weight, row
        //      G <= c < 2G -> fp16 lo of head c - G's weight.  Slot i = token
        //      t0 + 16 (i / 4) + 4 grp + i % 4, the same slots V uses below.
        half8 pa;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = t0 + 16 * (i >> 2) + 4 * grp + (i & 3);
            const float vscale = tok < t_end ? vsb[(int64_t)tok * Hkv] : 0.0f;
            const float w = p[i] * vscale * p2;
            const float wo = __shfl_up(w, G, 16);
            _Float16 h, l;
            split_one(c < G ? w : wo, h, l);
            pa[i] = c < G ? h : (c < 2 * G ? l : (_Float16)0.0f);
        }
        // rescale the running output rows by their head's alpha
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * grp + e;
            const int hr = r < G ? r : (r < 2 * G ? r - G : 0);
            const float ar = __shfl(alpha, hr, 64);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt][e] *= (r < 2 * G ? ar : 0.0f);
        }

        // ---- V tile into LDS, then 8 d-tiles of 16 ---------------------------
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int chunk = lane + 64 * i;
            *reinterpret_cast<uint4*>(vt + (chunk >> 4) * VROW + (chunk & 15) * 16) = vraw[i];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int d = 16 * dt + c;
            uint4 raw;
            uint32_t w[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i0 = 2 * jj, i1 = 2 * jj + 1;
                const int r0 = 16 * (i0 >> 2) + 4 * grp + (i0 & 3);
                const int r1 = 16 * (i1 >> 2) + 4 * grp + (i1 & 3);
                const uint16_t a0 = *reinterpret_cast<const uint16_t*>(vt + r0 * VROW + 2 * d);
                const uint16_t a1 = *reinterpret_cast<const uint16_t*>(vt + r1 * VROW + 2 * d);
                w[jj] = (uint32_t)a0 | ((uint32_t)a1 << 16);
            }
            raw = make_uint4(w[0], w[1], w[2], w[3]);
            half8 vh, vl;
            unpack8(raw, vh, vl);
            mfma16(pa, vh, acc[dt]);
            mfma16(pa, vl, acc[dt]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- write this range's (m, l, o): o[h][d] = row h + row (G + h) / 2^10,
    //      divided by the power of two folded into the weights -----------------
    float* ob = reinterpret_cast<float*>(vt);        // [2G][D] staging, reuses the V tile
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * grp + e;
            if (r < 2 * G) ob[r * D + 16 * dt + c] = acc[dt][e];
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

// Merge the ranges of one (b, h) in range order: out = sum_u w_u o_u / sum_u w_u l_u,
// w_u = exp(m_u - max_u m_u).
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part,
                                                           float* __restrict__ out, int Hq, int Hkv,
                                                           int G, int units) {
    const int bh = blockIdx.x;
    const int b = bh / Hq, h = bh - b * Hq;
    const int gk = h / G, c = h - gk * G;
    const int d = threadIdx.x;
    const int64_t stride = 2 * G + G * D;
    const float* base = part + ((int64_t)b * Hkv + gk) * units * stride;
    float M = -INFINITY;
    for (int u = 0; u < units; ++u) M = fmaxf(M, base[u * stride + c]);
    float L = 0.0f, O = 0.0f;
    for (int u = 0; u < units; ++u) {
        const float* pu = base + u * stride;
        const float w = expf(pu[c] - M);
        L += w * pu[G + c];
        O += w * pu[2 * G + c * D + d];
    }
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

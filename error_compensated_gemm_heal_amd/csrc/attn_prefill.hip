// Prefill (causal self-) attention over INT16 Q/K/V, with the INT16 ->
// dual-FP16 unpack fused into the operand loads.
//
// HEAL paper, section 3, "Mitigating QKV Truncation Error via INT16
// Quantization": Q, K and V are stored as INT16 codes with one scale per
// token and head, and attention runs as 16-bit products of the codes' exact
// FP16 parts with FP32 accumulation.  For a prompt of T tokens, query t
// attends keys 0 .. t.
//
// Codes split as q = 64 qh + ql, qh = q >> 6 in [-512, 511], ql = q & 63;
// qh, 64 qh and ql are exact FP16 values, and every product formed below is
// exact in FP32 (at most 22 significant bits).
//
// One block of 8 waves owns 128 consecutive queries of one (batch, head);
// wave w takes queries 16 w .. 16 w + 15 of them.  The block walks the key
// blocks of 64 tokens that its queries can see (causal); a wave computes the
// ones its own queries see, so the first four waves skip the block's last
// key block.  Each thread loads its share of the next block's K and V codes
// into registers while the current block is computed, and unpacks it into
// fp16 planes in LDS (K hi and 64 V hi exact, lo biased) once for all eight waves;
// two sets of planes alternate, so one barrier per key block suffices:
//  * scores as S^T = K . Q^T on v_mfma_f32_16x16x32_f16: rows are keys,
//    columns the wave's 16 queries.  A = {kh, kl + 1024}, B = {64 qh, ql}: the
//    kh products go to one accumulator, the biased kl products to a second
//    one that starts from -1024 sum_d (64 qh + ql) (an MFMA against a constant
//    -1024 operand, once per wave), and k . q = 64 S_hi + S_lo.  The biased low
//    half is one bit operation per two codes;
//  * online softmax in base 2 (log2 e folded into s_q s_k / sqrt(D)): per
//    query the running maximum, the running sum, and the output rescaled by
//    2^(m_old - m_new) when the maximum moves;
//  * P . V: the S^T register layout is the A-operand layout of P (lane =
//    query), so P needs no transpose.  A key's weight p_t s_v(t) 2^E (2^E a
//    power of two per key block keeping the weights below 2) is split into
//    fp16 hi + lo 2^-10; V comes from LDS through the transposing
//    ds_read_b64_tr_b16 on the V planes as {vh, vl + 1024}; the weight
//    x = p s_v 2^(9 - E) splits into fp16 H + L, which enter one fresh
//    accumulator against the planes {64 vh, vl + 1024},
//    started from -1024 times the weight sums to cancel the bias; the output
//    is held in units of the block factor 2^(E - 9) and merged as
//    acc 2^(m_old - m_new) 2^(E_old - E) + block.
#include <type_traits>

#include "heal_internal.h"

namespace heal {

namespace {

constexpr int D = 128;
constexpr int QW = 16;                // queries per wave
constexpr int WPB = 8;                // waves per block
constexpr int QB = QW * WPB;          // queries per block
constexpr int KB = 64;                // keys per step
constexpr int PLANE = KB * D * 2;     // LDS bytes of one fp16 plane of a K or V tile
constexpr int KH = 0, KL = PLANE, VH = 2 * PLANE, VL = 3 * PLANE;   // plane offsets in one set
constexpr int BUF = 4 * PLANE;        // one set of the four planes (64 KB)
constexpr int RPS = 64 * WPB / 16;    // token rows one pass of the block's threads covers
constexpr int SHARE = KB / RPS;       // 16-byte chunks per thread per K (or V) tile
static_assert(QB % KB == 0 && KB % QW == 0 && KB % RPS == 0, "tiling");
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

// 8 int16 codes (4 dwords) -> exact fp16 parts (code >> 6) and (code & 63).
// code >> 6 lies in [-512, 511]: adding the fp16 pattern 0x6600 gives the fp16
// number 1536 + (code >> 6) in [1024, 2047], where fp16 spacing is 1, and
// subtracting 1536 leaves it exactly.  code & 63 or'ed into 0x6400 is the fp16
// number 1024 + (code & 63).
__device__ __forceinline__ void unpack8(const u32x4& raw, half8& hi, half8& lo) {
    u32x4 hw, lw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = raw[i];
        const short2v t = __builtin_bit_cast(short2v, w) >> (short2v)(short)6;
        const ushort2v u = __builtin_bit_cast(ushort2v, t) + (ushort2v)(unsigned short)0x6600;
        hw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, u) - (half2v)(_Float16)1536.0f);
        lw[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, (w & 0x003F003Fu) | 0x64006400u) -
                                                 (half2v)(_Float16)1024.0f);
    }
    hi = __builtin_bit_cast(half8, hw);
    lo = __builtin_bit_cast(half8, lw);
}
// The same high halves; the low halves left biased, as the fp16 numbers
// 1024 + (code & 63), in one bit operation ((w & 0x003F003F) | 0x64006400).
// A product chain over biased low halves starts from -1024 times the sum of
// the other operand, which removes the bias; every product stays exact.
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

// Reductions over the lanes that share lane % 16 (one query column).
__device__ __forceinline__ float group_max(float x) {
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
// x of lane `src` (a lane-index permute; no LDS memory is touched)
__device__ __forceinline__ float from_lane(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

// LDS placement: token row r of a K tile holds its sixteen 16-byte chunks in
// slots chunk ^ (r % 16), so 16 lanes reading one chunk of 16 rows hit 16
// distinct slots; a V tile uses chunk ^ 2 (r % 8), which the transposing reads
// need (as in the decode kernel).
__device__ __forceinline__ int kswz(int r) { return r & 15; }
__device__ __forceinline__ int vswz(int r) { return 2 * (r & 7); }

__global__ __launch_bounds__(64 * WPB) void attn_prefill_kernel(
    const int16_t* __restrict__ q, const float* __restrict__ qs, const int16_t* __restrict__ k,
    const float* __restrict__ ks, const int16_t* __restrict__ v, const float* __restrict__ vs,
    float* __restrict__ out, int T, int Hq, int Hkv, int nqb, int nbh) {
    // two sets of planes: the waves compute on one while the next key
    // block is unpacked into the other
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * BUF];
    // per set: the key block's K and V scales and its block factor's
    // exponent E - 9, written once by wave 0
    __shared__ __attribute__((aligned(16))) float sks[2][KB], svs[2][KB];
    __shared__ int sbeta[2];
    const int lane = threadIdx.x & 63;
    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // heavy (late) query blocks first over all (batch, head) pairs: they see
    // the most keys, and the light ones fill the tail
    const int bh = (int)(blockIdx.x % nbh);
    const int qb = nqb - 1 - (int)(blockIdx.x / nbh);
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int G = Hq / Hkv;
    const int gk = h / G;
    const int c = lane & 15, grp = lane >> 4;
    const int q0 = qb * QB + wid * QW;          // the wave's first query
    const int qi = q0 + c;                      // this lane's query column
    const int nkb_t = (T + KB - 1) / KB;        // key blocks of the prompt
    // key blocks the block walks (up to the diagonal of its last query), and
    // those this wave computes: up to the one holding its own queries (no
    // wave's 16 queries straddle two key blocks); none for a wave wholly past T
    const int nkb = min((qb * QB + QB - 1) / KB + 1, nkb_t);
    const int nkb_w = q0 < T ? min((q0 + QW - 1) / KB + 1, nkb_t) : 0;
    const uint32_t row_bytes = (uint32_t)Hkv * D * 2;  // bytes between tokens in the cache

    // ---- Q as the B operand: lane (c, grp) holds query qi, d = 32 s + 8 grp + j
    half8 qh[4], ql[4];
    {
        const bool ok = qi < T;
        const int16_t* qrow = q + (((int64_t)b * T + (ok ? qi : 0)) * Hq + h) * D;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * grp);
            if (!ok) raw = (u32x4){0u, 0u, 0u, 0u};
            half8 hi;
            unpack8(raw, hi, ql[s]);
            qh[s] = hi * (_Float16)64.0f;   // exact: |64 qh| <= 32768
        }
    }
    // start of the biased kl chains: -1024 sum_d (64 qh + ql) of query column c
    floatx4 qbias = {0.f, 0.f, 0.f, 0.f};
    {
        const half8 m1024 = (half8)(_Float16)-1024.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            mfma16(m1024, qh[s], qbias);
            mfma16(m1024, ql[s], qbias);
        }
    }
    const float qscale = qi < T ? qs[((int64_t)b * T + qi) * Hq + h] * kLog2eInvSqrtD : 0.0f;

    // ---- this thread's share of a K (or V) tile: the 16-byte chunks
    //      tid + 64 WPB i, i.e. token row RPS i + tid / 16, chunk tid % 16,
    //      loaded into registers and unpacked into the planes at the tile's
    //      swizzled slots.  Tokens past T, and blocks past the last one the
    //      block walks, read as zero (an empty buffer range: no memory is
    //      touched), so the loads of a block ahead need no condition.
    const int sh_row = tid >> 4, sh_chunk = tid & 15;
    u32x4 rk[SHARE], rv[SHARE];
    auto load_raw = [&](int kb) {
        const int t0 = min(kb, nkb - 1) * KB;
        const int nt = kb < nkb ? __builtin_amdgcn_readfirstlane(min(KB, T - t0)) : 0;
        const int64_t tok0 = ((int64_t)b * T + t0) * Hkv + gk;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + tok0 * D, (uint32_t)nt * row_bytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + tok0 * D, (uint32_t)nt * row_bytes);
#pragma unroll
        for (int i = 0; i < SHARE; ++i) {
            const uint32_t off = (uint32_t)(RPS * i + sh_row) * row_bytes + 16u * (uint32_t)sh_chunk;
            rk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
            rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
        }
    };
    auto write_planes = [&](unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < SHARE; ++i) {
            const int row = RPS * i + sh_row;
            half8 hi, lo;
            unpack8_lobias(rk[i], hi, lo);
            const int ko = row * (D * 2) + 16 * (sh_chunk ^ kswz(row));
            *reinterpret_cast<half8*>(buf + KH + ko) = hi;
            *reinterpret_cast<half8*>(buf + KL + ko) = lo;
            unpack8_lobias(rv[i], hi, lo);
            const int vo = row * (D * 2) + 16 * (sh_chunk ^ vswz(row));
            *reinterpret_cast<half8*>(buf + VH + vo) = hi * (_Float16)64.0f;   // exact: |64 vh| <= 32768
            *reinterpret_cast<half8*>(buf + VL + vo) = lo;
        }
    };
    // scales of a block's keys: lane t of wave 0 loads key t's K and V scales
    // (0 past T, and past the last block) and, once the block's planes are
    // written, puts them in the block's set with E - 9, E the exponent of
    // the largest V scale of the block's 64 keys (so s_v(t) 2^(9 - E) lies
    // in [0, 512)); every wave then reads them from LDS instead of loading
    // and reducing them itself
    float ks_r = 0.0f, vs_r = 0.0f;
    auto load_scales = [&](int kb) {
        if (wid != 0) return;
        const int t0 = min(kb, nkb - 1) * KB;
        const int nt = kb < nkb ? __builtin_amdgcn_readfirstlane(min(KB, T - t0)) : 0;
        const int64_t tok0 = ((int64_t)b * T + t0) * Hkv + gk;
        const uint32_t srec = nt > 0 ? (uint32_t)(((nt - 1) * Hkv + 1) * 4) : 0u;
        const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(ks + tok0, srec);
        const __amdgpu_buffer_rsrc_t vsrs = make_rsrc(vs + tok0, srec);
        const uint32_t off = (uint32_t)(lane * Hkv * 4);
        ks_r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksrs, off, 0, 0));
        vs_r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsrs, off, 0, 0));
    };
    auto write_scales = [&](int set) {
        if (wid != 0) return;
        const float vmax = max_swap32(max_half(vs_r));
        int vexp = 0;
        (void)frexpf(vmax, &vexp);
        const int ebeta = vmax > 0.0f ? vexp - 9 : 0;
        sks[set][lane] = ks_r;
        svs[set][lane] = vs_r;
        if (lane == 0) sbeta[set] = ebeta;
    };

    // ---- running softmax state of query column c (the same on its 4 lanes)
    //      and the output: lane (c, grp) holds d = 16 dt + c of queries
    //      q0 + 4 grp + e in acc[dt][e]
    float m_run = -INFINITY, l_run = 0.0f;
    int ebeta_run = 0;       // the output's current block factor 2^ebeta_run (acc holds out / 2^ebeta_run)
    floatx4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = (floatx4){0.f, 0.f, 0.f, 0.f};

    // one key block from the planes at buf; only the wave's last one (its
    // diagonal, or the ragged end of the prompt) has keys a query of the wave
    // may not see
    auto key_block = [&](int kb, const unsigned char* buf, int set, auto masked) {
        // the block's scales where the score layout needs them: index 4 st + e
        // is key 16 st + 4 grp + e
        float ksv[16], vsv[16];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const float4 k4 = *reinterpret_cast<const float4*>(&sks[set][16 * st + 4 * grp]);
            const float4 v4 = *reinterpret_cast<const float4*>(&svs[set][16 * st + 4 * grp]);
            ksv[4 * st] = k4.x; ksv[4 * st + 1] = k4.y; ksv[4 * st + 2] = k4.z; ksv[4 * st + 3] = k4.w;
            vsv[4 * st] = v4.x; vsv[4 * st + 1] = v4.y; vsv[4 * st + 2] = v4.z; vsv[4 * st + 3] = v4.w;
        }
        const int ebeta = sbeta[set];
        const float p2 = ldexpf(1.0f, -ebeta);
        // ---- scores: sc[4 st + e] for key 16 st + 4 grp + e of the block
        float sc[16];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            floatx4 s_hi = {0.f, 0.f, 0.f, 0.f}, s_lo = qbias;
            const int row = 16 * st + c;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ko = row * (D * 2) + 16 * ((4 * s + grp) ^ kswz(row));
                const half8 kh = *reinterpret_cast<const half8*>(buf + KH + ko);
                const half8 klb = *reinterpret_cast<const half8*>(buf + KL + ko);
                mfma16(kh, qh[s], s_hi);
                mfma16(kh, ql[s], s_hi);
                mfma16(klb, qh[s], s_lo);
                mfma16(klb, ql[s], s_lo);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[4 * st + e] = (64.0f * s_hi[e] + s_lo[e]) * (qscale * ksv[4 * st + e]);
                if constexpr (decltype(masked)::value) {
                    // an added -inf rather than a branch (the score is finite)
                    const int key = kb * KB + 16 * st + 4 * grp + e;
                    sc[4 * st + e] += (key <= qi && key < T) ? 0.0f : -INFINITY;
                }
            }
        }
        float mb = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mb = fmaxf(mb, sc[i]);
        mb = group_max(mb);
        const float m_new = fmaxf(m_run, mb);
        // m_new is finite: every key of an unmasked block is visible, and the
        // first key of the wave's last block is visible to every query of the
        // wave (and lies before T).  exp2(-inf) = 0 covers the first block's
        // alpha and the masked scores.
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[16], psum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
            psum += p[i];
        }
        l_run = l_run * alpha + group_sum(psum);
        m_run = m_new;

        // x = p s_v(t) 2^(9 - E) lies in [0, 512); its block factor 2^(E - 9)

        // ---- P as the A operand for key halves kh2 = 0, 1 (32 keys each):
        //      slot i = key 32 kh2 + 16 (i / 4) + 4 grp + i % 4.  The weight
        //      x splits as H = fp16(x), L = fp16(x - H) (x - H is exact in fp32;
        //      H + L holds x to 2^-22, and L keeps it in normal range down to
        //      x ~ 2^-3, to 2^-24 absolute below); with V's parts v = 64 vh + vl
        //      the operands are H and L against the plane of 64 vh (|64 vh| <=
        //      2^15, exact), and against vl.  Every product is exact.
        half8 pa_h[2], pa_l[2];
#pragma unroll
        for (int kh2 = 0; kh2 < 2; ++kh2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = p[8 * kh2 + i] * vsv[8 * kh2 + i] * p2;
                const _Float16 hh = (_Float16)x;
                pa_h[kh2][i] = hh;
                pa_l[kh2][i] = (_Float16)(x - (float)hh);
            }
        }

        // ---- P . V into a fresh accumulator; V by transposing LDS reads: in
        //      each 16-lane group, lane 4 j + x supplies the address of 4 d at
        //      16 dt + 4 x of token row 4 grp + j (+ 16 half + 32 kh2); lane i
        //      receives d = 16 dt + i of those 4 tokens
        // the biased vl products start from -1024 times the block's weight sums
        floatx4 bias = {0.f, 0.f, 0.f, 0.f};
        {
            const half8 m1024 = (half8)(_Float16)-1024.0f;
#pragma unroll
            for (int kh2 = 0; kh2 < 2; ++kh2) {
                mfma16(pa_h[kh2], m1024, bias);
                mfma16(pa_l[kh2], m1024, bias);
            }
        }
        floatx4 blk[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) blk[dt] = bias;
        {
            const int s16 = lane & 15;
            const int rr = 4 * grp + (s16 >> 2);
            const int lane_off = rr * (D * 2) + 16 * ((s16 & 3) >> 1) + 8 * (s16 & 1);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int off = lane_off + 16 * ((2 * dt) ^ vswz(rr));
#pragma unroll
                for (int kh2 = 0; kh2 < 2; ++kh2) {
                    const int o0 = off + (32 * kh2) * (D * 2), o1 = off + (32 * kh2 + 16) * (D * 2);
                    const u32x2 h0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(buf + VH + o0)));
                    const u32x2 h1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(buf + VH + o1)));
                    const u32x2 l0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(buf + VL + o0)));
                    const u32x2 l1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(buf + VL + o1)));
                    const half8 vh64 = __builtin_bit_cast(half8, (u32x4){h0.x, h0.y, h1.x, h1.y});
                    const half8 vlb = __builtin_bit_cast(half8, (u32x4){l0.x, l0.y, l1.x, l1.y});
                    mfma16(pa_h[kh2], vh64, blk[dt]);
                    mfma16(pa_h[kh2], vlb, blk[dt]);
                    mfma16(pa_l[kh2], vh64, blk[dt]);
                    mfma16(pa_l[kh2], vlb, blk[dt]);
                }
            }
        }
        // ---- the output is kept in units of the current block factor:
        //      out = acc beta, so acc <- acc alpha (beta_old / beta) + blk (the
        //      ratio is a power of two, exact); lane (c, grp) holds the rows of
        //      queries 4 grp + e, whose alpha sits on lane 4 grp + e
        const float ratio = ldexpf(1.0f, ebeta_run - ebeta);
        ebeta_run = ebeta;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f_e = from_lane(alpha, 4 * grp + e) * ratio;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt][e] = __builtin_fmaf(acc[dt][e], f_e, blk[dt][e]);
        }
    };

    // block 0 unpacked into the first planes; block 1's codes and block 0's
    // scales in flight
    load_raw(0);
    load_scales(0);
    write_planes(lds);
    write_scales(0);
    load_raw(1);
    load_scales(1);
    for (int kb = 0; kb < nkb; ++kb) {
        // block kb's planes and scales are complete, and every wave is done
        // with block kb - 1, whose set block kb + 1 now takes
        __syncthreads();
        unsigned char* cur = lds + (kb & 1) * BUF;
        unsigned char* nxt = lds + ((kb + 1) & 1) * BUF;
        if (kb + 1 < nkb_w) key_block(kb, cur, kb & 1, std::false_type{});
        else if (kb + 1 == nkb_w) key_block(kb, cur, kb & 1, std::true_type{});
        if (kb + 1 < nkb) {
            write_planes(nxt);
            write_scales((kb + 1) & 1);
        }
        load_raw(kb + 2);
        load_scales(kb + 2);
    }

    // ---- normalize and store: rows q0 + 4 grp + e, d = 16 dt + c
    if (nkb_w > 0) {
        const float beta_run = ldexpf(1.0f, ebeta_run);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float l_e = from_lane(l_run, 4 * grp + e);
            const int qrow = q0 + 4 * grp + e;
            if (qrow < T) {
                float* o = out + (((int64_t)b * T + qrow) * Hq + h) * D + c;
                const float inv = 1.0f / l_e;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[16 * dt] = acc[dt][e] * beta_run * inv;
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_prefill(const int16_t* q, const float* qs, const int16_t* k, const float* ks,
                               const int16_t* v, const float* vs, float* out, int64_t B, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t Dd, hipStream_t s) {
    if (Dd != D) return hipErrorInvalidValue;
    const int nqb = (int)((T + QB - 1) / QB);
    const unsigned blocks = (unsigned)(B * Hq * nqb);
    hipLaunchKernelGGL(attn_prefill_kernel, dim3(blocks), dim3(64 * WPB), 0, s, q, qs, k, ks, v, vs, out, (int)T,
                       (int)Hq, (int)Hkv, nqb, (int)(B * Hq));
    return hipGetLastError();
}

}  // namespace heal

// fp8 (OCP E4M3) quantisation of packed Q, K and V with power-of-two dequantisation
// scales, and the channel split of the corrected mode.
//
// The VisualGen FLUX 3 article (everytik.com translation, section 量化注意力与稀疏注意力)
// runs attention with fp8 Q/K and V; block-wise scale factors follow the kongchang.com
// English page (section "Reducing Numerical Precision").  Granularity: Q and K one scale
// per (b, h, 128 packed tokens), V one scale per (b, h, channel).  Every scale is the
// smallest power of two s with amax <= 448 s (as the shared scales of the OCP MX
// formats), so x / s is exact and the e4m3 rounding (nearest, ties to even) is the only
// rounding: codes are bit-exact by construction.
//
// Corrected mode: per (b, h) the 16 channels with the largest amax|q_c| * amax|k_c|
// (ties to the lower index) are kept out of the e4m3 product.  Their e4m3 codes are
// written as zero and their exact values divided by the block scale are written as bf16
// (exact: a power-of-two rescale of a bf16 value), to be accumulated by a bf16 MFMA next
// to the fp8 ones.
//
// The streams variant (GATHER) reads Q, K and V in place from the per-stream tensors: Q/K
// blocks as above (row by row where a block straddles two streams); V, whose scale spans
// all tokens and whose output is channel-major, through a block-parallel channel amax and
// a 64-token tile kernel that quantises and transposes through LDS.
//
// Token repair (the repair budget of VC-Attention FP8, same article section): the plain
// codes, plus per token the largest absolute residual |x - decode(code) * scale| over the
// head's channels (exact in binary32: a bf16 value minus its e4m3 neighbour times a power
// of two), and per (b, h) the n tokens of largest residual (ties to the lower index),
// found by a 4-pass radix select over the residuals' bit patterns and listed in
// ascending order by an ordered compaction.
//
// All kernels are bound by HBM bandwidth.  One workgroup owns one scale segment, which
// is contiguous in the layouts used here (a 128-token block of a BHND tensor is
// 128 * D consecutive elements; a V channel is one BHDN row): pass 1 takes the absolute
// maximum, pass 2 re-reads the segment (now in L2) and writes the codes.
#include "ja_device.h"
#include "ja_launch.h"

namespace ja {
namespace {

constexpr int NT = 256;

// finite binary32 -> e4m3 code, round to nearest even, saturating at +-448 (written from
// the OCP E4M3 definition: bias 7, 3 mantissa bits, subnormal step 2^-9)
__device__ inline uint32_t e4m3_from_f32(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.0f);
    uint32_t code;
    if (a >= 0.015625f) {                              // normal range, >= 2^-6
        const uint32_t u = __float_as_uint(a);
        // keep 3 of the 23 mantissa bits, ties to even; a carry bumps the exponent
        const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
        code = r - ((127u - 7u) << 3);                 // rebias the exponent 127 -> 7
    } else {                                           // subnormal: multiples of 2^-9
        code = (uint32_t)rintf(a * 512.0f);            // exact product, ties to even
    }
    return code | sign;
}

// e4m3 code -> binary32 value, exact (written from the same definition)
__device__ inline float f32_from_e4m3(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float a = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -a : a;
}

// smallest k >= -126 with amax <= 448 * 2^k (k = 0 for amax == 0).  With
// amax = (1 + m / 2^23) * 2^(e - 127): 448 * 2^(e-135) = 1.75 * 2^(e-127), so k = e - 135
// when m <= 0.75 * 2^23 and e - 134 otherwise.
__device__ inline int pow2_exponent(float amax) {
    if (amax == 0.f) return 0;
    const uint32_t u = __float_as_uint(amax);
    const int e = (int)((u >> 23) & 0xFFu);
    if (e == 0) return -126;                           // denormal amax
    const int k = ((u & 0x7FFFFFu) <= 0x600000u) ? e - 135 : e - 134;
    return k < -126 ? -126 : k;
}

__device__ inline void bf16x2_to_f32(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
}

__device__ inline float block_max(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

// 8 bf16 (one uint4) -> 8 e4m3 codes (one uint2); `keep` bit e zeroes code e
__device__ inline uint2 quant8(uint4 v, float inv, uint32_t keep = 0) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo, hi;
        bf16x2_to_f32(w[e], lo, hi);
        uint32_t c0 = e4m3_from_f32(lo * inv), c1 = e4m3_from_f32(hi * inv);
        if (keep & (1u << (2 * e))) c0 = 0;
        if (keep & (2u << (2 * e))) c1 = 0;
        out[e / 2] |= (c0 | (c1 << 8)) << (16 * (e % 2));
    }
    return make_uint2(out[0], out[1]);
}

__device__ inline float amax8(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo, hi;
        bf16x2_to_f32(w[e], lo, hi);
        m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
    }
    return m;
}

// ---- where the rows of packed tokens come from: the packed tensor [B][H][N][D], or
//      (GATHER) the per-stream tensors [B][L_s][H][D] of a StreamTable
__device__ inline int stream_index(const StreamTable& st, int t) {
    int s = 0;
    for (int i = 1; i < st.n; ++i)
        if (t >= st.off[i]) s = i;                   // zero-length streams share the next start
    return s;
}

__device__ inline const uint16_t* stream_token_row(const StreamTable& st, const void* const* src,
                                                   int b, int h, int H, int D, int t) {
    const int s = stream_index(st, t);
    const int64_t L = st.off[s + 1] - st.off[s];
    return static_cast<const uint16_t*>(src[s]) +
           (((int64_t)b * L + (t - st.off[s])) * H + h) * (int64_t)D;
}

// rows of tokens t0 .. t0 + rows - 1 of one (b, h): one strided run (packed, or inside a
// single stream), else looked up row by row
struct RowMap {
    const uint16_t* run;     // row of t0, or nullptr
    int64_t pitch;           // elements between consecutive rows of the run
};

template <bool GATHER>
__device__ inline RowMap row_map(const uint16_t* packed_bh, const StreamTable& st,
                                 const void* const* src, int b, int h, int H, int D, int t0,
                                 int rows) {
    if (!GATHER) return {packed_bh + (int64_t)t0 * D, D};
    const int s = stream_index(st, t0);
    if (t0 + rows <= st.off[s + 1]) return {stream_token_row(st, src, b, h, H, D, t0), (int64_t)H * D};
    return {nullptr, 0};
}

__device__ inline const uint16_t* row_ptr(const RowMap& m, const StreamTable& st,
                                          const void* const* src, int b, int h, int H, int D,
                                          int t0, int r) {
    return m.run ? m.run + r * m.pitch : stream_token_row(st, src, b, h, H, D, t0 + r);
}

// corrected mode, step 0 -- clear ch_amax (a plain fill kernel, also safe under graph
// capture)
__global__ __launch_bounds__(NT) void clear_kernel(float* __restrict__ x, int n) {
    const int i = blockIdx.x * NT + threadIdx.x;
    if (i < n) x[i] = 0.f;
}

// corrected mode, step 1 -- grid (n_blocks, B*H, 2): per-channel amax of one 128-token
// block of Q (z = 0) or K (z = 1), folded into ch_amax [B, H, 2, D] with an atomic max on
// the bit patterns (non-negative floats order like their bits; max is order-free, so the
// result is deterministic).
template <int D, bool GATHER>
__global__ __launch_bounds__(NT) void chan_amax_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ k,
                                                      const StreamTable st, int H, int N,
                                                      float* __restrict__ ch_amax) {
    constexpr int CPR = D / 8;                        // 16-byte chunks per token row
    constexpr int RPP = NT / CPR;                     // rows handled in parallel
    __shared__ float part[RPP][D + 1];
    const int blk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const int t0 = blk * JA_QK_BLOCK;
    const int rows = min(JA_QK_BLOCK, N - t0);
    const int ch = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    const void* const* xs = blockIdx.z ? st.k : st.q;
    const RowMap rm = row_map<GATHER>((blockIdx.z ? k : q) + (int64_t)bh * N * D, st, xs, b, h,
                                      H, D, t0, rows);
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int row = r0; row < rows; row += RPP) {
        const uint4 v =
            *reinterpret_cast<const uint4*>(row_ptr(rm, st, xs, b, h, H, D, t0, row) + ch * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo, hi;
            bf16x2_to_f32(w[e], lo, hi);
            m[2 * e] = fmaxf(m[2 * e], fabsf(lo));
            m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(hi));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][ch * 8 + e] = m[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float mx = 0.f;
        for (int r = 0; r < RPP; ++r) mx = fmaxf(mx, part[r][threadIdx.x]);
        unsigned int* dst = reinterpret_cast<unsigned int*>(ch_amax) +
                            ((int64_t)bh * 2 + blockIdx.z) * D + threadIdx.x;
        atomicMax(dst, __float_as_uint(mx));
    }
}

// corrected mode, step 2 -- grid (B*H), one wave: the 16 channels with the largest
// amax_q * amax_k (exact: products of bf16 values), ascending order -> hi_idx.
template <int D>
__global__ __launch_bounds__(64) void select_hi_kernel(const float* __restrict__ ch_amax,
                                                      int32_t* __restrict__ hi_idx) {
    const int bh = blockIdx.x, lane = threadIdx.x;
    const float* qa = ch_amax + (int64_t)bh * 2 * D;
    const float* ka = qa + D;
    float sc[D / 64];
    bool taken[D / 64];
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        sc[j] = qa[lane + 64 * j] * ka[lane + 64 * j];
        taken[j] = false;
    }
    // 16 rounds of arg-max (ties to the lower index); every lane ends with the same list
    int chosen[JA_HI_CHANNELS];
#pragma unroll
    for (int round = 0; round < JA_HI_CHANNELS; ++round) {
        float best = -1.f;
        int bidx = D;
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
            const int c = lane + 64 * j;
            if (!taken[j] && (sc[j] > best || (sc[j] == best && c < bidx))) {
                best = sc[j];
                bidx = c;
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float ob = __shfl_xor(best, o);
            const int oi = __shfl_xor(bidx, o);
            if (ob > best || (ob == best && oi < bidx)) {
                best = ob;
                bidx = oi;
            }
        }
        chosen[round] = bidx;
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
            if (lane + 64 * j == bidx) taken[j] = true;
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 1; i < JA_HI_CHANNELS; ++i)          // ascending channel order
#pragma unroll
            for (int j = JA_HI_CHANNELS - 1; j >= i; --j)
                if (chosen[j - 1] > chosen[j]) {
                    const int t = chosen[j];
                    chosen[j] = chosen[j - 1];
                    chosen[j - 1] = t;
                }
#pragma unroll
        for (int i = 0; i < JA_HI_CHANNELS; ++i)
            hi_idx[(int64_t)bh * JA_HI_CHANNELS + i] = chosen[i];
    }
}

// grid: (n_blocks, B*H, 2) -- z selects Q (0) or K (1).  With hi_idx, the selected
// channels' codes are zero and their values / scale go to hi (bf16 [B, H, N, 16]).
// ERR: also each token's largest absolute residual -> q_err / k_err (fp32 [B, H, N]).
template <int D, bool SPLIT, bool GATHER, bool ERR = false>
__global__ __launch_bounds__(NT) void quant_qk_kernel(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     const StreamTable st, int H, int N,
                                                     uint8_t* __restrict__ q8,
                                                     uint8_t* __restrict__ k8,
                                                     float* __restrict__ qs,
                                                     float* __restrict__ ks, int nblk,
                                                     const int32_t* __restrict__ hi_idx,
                                                     uint16_t* __restrict__ q_hi,
                                                     uint16_t* __restrict__ k_hi,
                                                     float* __restrict__ q_err = nullptr,
                                                     float* __restrict__ k_err = nullptr) {
    static_assert(NT % (D / 8) == 0 && (JA_QK_BLOCK * D / 8) % NT == 0, "chunk mapping");
    __shared__ float red[NT / 64];
    __shared__ uint32_t mask[D / 32];
    // SPLIT: the block's kept values / scale, [row][rank of the channel among the kept]
    __shared__ uint4 hi_tab[SPLIT ? JA_QK_BLOCK * JA_HI_CHANNELS / 8 : 1];
    const uint16_t* x = blockIdx.z ? k : q;
    uint8_t* y = blockIdx.z ? k8 : q8;
    float* sc = blockIdx.z ? ks : qs;
    const int blk = blockIdx.x, bh = blockIdx.y;
    const int t0 = blk * JA_QK_BLOCK;
    const int rows = min(JA_QK_BLOCK, N - t0);
    const int64_t base = ((int64_t)bh * N + t0) * D;    // of the packed output block
    const int nch = rows * D / 8;                       // 16-byte input chunks in the segment
    const int b = bh / H, h = bh - b * H;
    const void* const* xs = blockIdx.z ? st.k : st.q;
    const RowMap rm = row_map<GATHER>(x + (int64_t)bh * N * D, st, xs, b, h, H, D, t0, rows);
    auto chunk = [&](int c) {                           // input chunk c of the block
        return *reinterpret_cast<const uint4*>(
            row_ptr(rm, st, xs, b, h, H, D, t0, c / (D / 8)) + (c % (D / 8)) * 8);
    };
    if (SPLIT) {
        if (threadIdx.x < D / 32) mask[threadIdx.x] = 0;
        __syncthreads();
        if (threadIdx.x < JA_HI_CHANNELS) {
            const int c = hi_idx[(int64_t)bh * JA_HI_CHANNELS + threadIdx.x];
            atomicOr(&mask[c / 32], 1u << (c % 32));
        }
    }

    // the block stays in registers between the amax and the encode pass
    constexpr int PER = JA_QK_BLOCK * D / 8 / NT;       // 16-byte chunks per thread
    uint4 reg[PER];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + i * NT;
        reg[i] = c < nch ? chunk(c) : make_uint4(0, 0, 0, 0);
        m = fmaxf(m, amax8(reg[i]));
    }
    const float amax = block_max(m, red);               // (its barrier also publishes mask)
    const int e = pow2_exponent(amax);
    const float inv = ldexpf(1.f, -e);
    if (threadIdx.x == 0) sc[(int64_t)bh * nblk + blk] = ldexpf(1.f, e);

    // NT is a multiple of D / 8, so a thread's chunks all cover the same 8 channels
    uint32_t keep = 0;
    int rank0 = 0;                                      // kept channels below this thread's 8
    if (SPLIT) {
        const int c0 = (threadIdx.x % (D / 8)) * 8;
        keep = (mask[c0 / 32] >> (c0 % 32)) & 0xFFu;
        for (int w = 0; w < c0 / 32; ++w) rank0 += __popc(mask[w]);
        rank0 += __popc(mask[c0 / 32] & ((1u << (c0 % 32)) - 1u));
    }
    uint2* dst = reinterpret_cast<uint2*>(y + base);
    const float scale = ldexpf(1.f, e);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int c = threadIdx.x + i * NT;
        const uint2 code = quant8(reg[i], inv, keep);
        if (c < nch) dst[c] = code;
        if (SPLIT && keep) {
            // hi_idx is ascending, so a kept channel's slot is its rank among the kept
            uint16_t* row = reinterpret_cast<uint16_t*>(hi_tab) + (c / (D / 8)) * JA_HI_CHANNELS;
            const uint32_t w[4] = {reg[i].x, reg[i].y, reg[i].z, reg[i].w};
            int j = rank0;
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2)
                if (keep & (1u << e2)) {
                    const float v = __uint_as_float(e2 % 2 ? w[e2 / 2] & 0xFFFF0000u : w[e2 / 2] << 16);
                    row[j++] = (uint16_t)(__float_as_uint(v * inv) >> 16);  // exact 2^-e rescale
                }
        }
        if constexpr (ERR) {
            // residuals of this chunk's 8 channels; the D / 8 chunks of a token sit in
            // D / 8 consecutive lanes of one wave
            const uint32_t w[4] = {reg[i].x, reg[i].y, reg[i].z, reg[i].w};
            const uint32_t cw[2] = {code.x, code.y};
            float r = 0.f;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float lo, hi;
                bf16x2_to_f32(w[e2], lo, hi);
                const uint32_t pair = cw[e2 / 2] >> (16 * (e2 % 2));
                r = fmaxf(r, fabsf(lo - f32_from_e4m3(pair & 0xFFu) * scale));
                r = fmaxf(r, fabsf(hi - f32_from_e4m3((pair >> 8) & 0xFFu) * scale));
            }
#pragma unroll
            for (int o = 1; o < D / 8; o <<= 1) r = fmaxf(r, __shfl_xor(r, o));
            if (c < nch && (threadIdx.x % (D / 8)) == 0)
                (blockIdx.z ? k_err : q_err)[(int64_t)bh * N + t0 + c / (D / 8)] = r;
        }
    }
    if (SPLIT) {
        // rows x 16 values, contiguous in q_hi / k_hi: copied out 16 bytes a lane
        __syncthreads();
        uint4* hi = reinterpret_cast<uint4*>((blockIdx.z ? k_hi : q_hi) +
                                             ((int64_t)bh * N + t0) * JA_HI_CHANNELS);
        for (int i = threadIdx.x; i < rows * JA_HI_CHANNELS / 8; i += NT) hi[i] = hi_tab[i];
    }
}

// grid: (D, B*H) -- one V^T row (b, h, channel) per workgroup.  The first VCACHE chunks
// per thread stay in registers between the two passes; longer rows re-read the rest.
constexpr int VCACHE = 9;                    // 2048x2048 rows (N = 16896) fit

__device__ inline uint4 v_chunk_masked(const uint4* src, int i, int nfull, int rem) {
    // chunk i of the row with the elements at or past N zeroed (zero encodes as code 0)
    uint4 v = src[i];
    if (i == nfull) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (2 * q >= rem) w[q] = 0;
            else if (2 * q + 1 >= rem) w[q] &= 0xFFFFu;
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return v;
}

__global__ __launch_bounds__(NT) void quant_v_kernel(const uint16_t* __restrict__ vt, int N,
                                                    int D, int64_t ldv,
                                                    uint8_t* __restrict__ v8t,
                                                    float* __restrict__ vs) {
    __shared__ float red[NT / 64];
    const int c = blockIdx.x, bh = blockIdx.y;
    const int64_t base = ((int64_t)bh * D + c) * ldv;
    const uint4* src = reinterpret_cast<const uint4*>(vt + base);
    const int nfull = N / 8;                           // chunks entirely inside [0, N)
    const int rem = N - nfull * 8;
    const int nval = nfull + (rem ? 1 : 0);            // chunks holding data
    const int nch = (int)(ldv / 8);                    // chunks in the padded row

    uint4 reg[VCACHE];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < VCACHE; ++j) {
        const int i = threadIdx.x + j * NT;
        reg[j] = i < nval ? v_chunk_masked(src, i, nfull, rem) : make_uint4(0, 0, 0, 0);
        m = fmaxf(m, amax8(reg[j]));
    }
    for (int i = threadIdx.x + VCACHE * NT; i < nval; i += NT)
        m = fmaxf(m, amax8(v_chunk_masked(src, i, nfull, rem)));
    const float amax = block_max(m, red);
    const int e = pow2_exponent(amax);
    const float inv = ldexpf(1.f, -e);
    if (threadIdx.x == 0) vs[(int64_t)bh * D + c] = ldexpf(1.f, e);

    uint2* dst = reinterpret_cast<uint2*>(v8t + base);
#pragma unroll
    for (int j = 0; j < VCACHE; ++j) {
        const int i = threadIdx.x + j * NT;
        if (i < nch) dst[i] = i < nval ? quant8(reg[j], inv) : make_uint2(0, 0);
    }
    for (int i = threadIdx.x + VCACHE * NT; i < nch; i += NT)
        dst[i] = i < nval ? quant8(v_chunk_masked(src, i, nfull, rem), inv) : make_uint2(0, 0);
}

// GATHER V, pass 1 -- grid (ceil(N / 256), B*H): per-channel amax of 256 tokens, folded
// into vmax [B][H][D] (the v_scale buffer, cleared first) with an atomic max on the bits.
template <int D>
__global__ __launch_bounds__(NT) void v_amax_kernel(const StreamTable st, int H, int N,
                                                   float* __restrict__ vmax) {
    constexpr int CPR = D / 8, RPP = NT / CPR, TT = 256;
    __shared__ float part[RPP][D + 1];
    const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
    const int t0 = blockIdx.x * TT, rows = min(TT, N - t0);
    const int ch = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    const RowMap rm = row_map<true>(nullptr, st, st.v, b, h, H, D, t0, rows);
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = r0; r < rows; r += RPP) {
        const uint4 v =
            *reinterpret_cast<const uint4*>(row_ptr(rm, st, st.v, b, h, H, D, t0, r) + ch * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo, hi;
            bf16x2_to_f32(w[e], lo, hi);
            m[2 * e] = fmaxf(m[2 * e], fabsf(lo));
            m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(hi));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][ch * 8 + e] = m[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float mx = 0.f;
        for (int r = 0; r < RPP; ++r) mx = fmaxf(mx, part[r][threadIdx.x]);
        atomicMax(reinterpret_cast<unsigned int*>(vmax) + (int64_t)bh * D + threadIdx.x,
                  __float_as_uint(mx));
    }
}

// GATHER V, pass 2 -- grid (ceil(ldv / 64), B*H): a 64-token tile quantised with the
// per-channel scales of pass 1 and transposed through LDS into 64-byte runs of the V^T
// code rows; tokens at or past N (the padding up to ldv) are written as code 0.
template <int D>
__global__ __launch_bounds__(NT) void quant_vt_kernel(const StreamTable st, int H, int N,
                                                     int64_t ldv, const float* __restrict__ vmax,
                                                     uint8_t* __restrict__ v8t) {
    constexpr int T = 64, CPR = D / 8, PITCH = T + 4;   // codes, channel-major
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    __shared__ float inv_s[D];
    const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
    const int t0 = blockIdx.x * T;
    const int rows = max(0, min(T, N - t0));
    for (int c = threadIdx.x; c < D; c += NT)
        inv_s[c] = ldexpf(1.f, -pow2_exponent(vmax[(int64_t)bh * D + c]));
    __syncthreads();
    const RowMap rm = row_map<true>(nullptr, st, st.v, b, h, H, D, t0, max(rows, 1));
    for (int x = threadIdx.x; x < T * CPR; x += NT) {
        const int r = x / CPR, col = x % CPR;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < rows)
            v = *reinterpret_cast<const uint4*>(row_ptr(rm, st, st.v, b, h, H, D, t0, r) +
                                                col * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo, hi;
            bf16x2_to_f32(w[e], lo, hi);
            const int c = col * 8 + 2 * e;
            tile[c * PITCH + r] = (uint8_t)e4m3_from_f32(lo * inv_s[c]);
            tile[(c + 1) * PITCH + r] = (uint8_t)e4m3_from_f32(hi * inv_s[c + 1]);
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < D * (T / 16); x += NT) {
        const int c = x / (T / 16), seg = x % (T / 16);
        const int64_t col0 = t0 + seg * 16;
        if (col0 < ldv) {                                // ldv % 16 == 0: whole 16-byte runs
            const uint32_t* src = reinterpret_cast<const uint32_t*>(&tile[c * PITCH + seg * 16]);
            *reinterpret_cast<uint4*>(v8t + ((int64_t)bh * D + c) * ldv + col0) =
                make_uint4(src[0], src[1], src[2], src[3]);
        }
    }
}

// GATHER V, pass 3: amax -> power-of-two scale, in place
__global__ __launch_bounds__(NT) void v_scale_final_kernel(float* __restrict__ vs, int n) {
    const int i = blockIdx.x * NT + threadIdx.x;
    if (i < n) vs[i] = ldexpf(1.f, pow2_exponent(vs[i]));
}

// Token repair: per (b, h) (blockIdx.x) and operand (blockIdx.y: Q, K), the n tokens of
// largest residual, ties to the lower index, in ascending order.  The residuals are
// non-negative floats, whose bit patterns order as integers: four 8-bit radix passes
// (per-wave histograms, summed per bin) find the n-th largest pattern T and how many
// tokens equal to T are taken (`need`); an ordered compaction then takes every token
// above T and the first `need` at T.  Requires 1 <= n <= N.
constexpr int SNT = 1024;
__global__ __launch_bounds__(SNT) void select_repair_kernel(const float* __restrict__ q_err,
                                                           const float* __restrict__ k_err,
                                                           int N, int n,
                                                           int32_t* __restrict__ q_sel,
                                                           int32_t* __restrict__ k_sel) {
    constexpr int NWV = SNT / 64;
    __shared__ uint32_t hist[NWV][256];
    __shared__ uint32_t total[256];
    __shared__ uint32_t sh_prefix, sh_need;
    __shared__ int wave_take[NWV], wave_eq[NWV];
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t* e = reinterpret_cast<const uint32_t*>((blockIdx.y ? k_err : q_err) +
                                                          (int64_t)bh * N);
    int32_t* out = (blockIdx.y ? k_sel : q_sel) + (int64_t)bh * n;

    uint32_t prefix = 0, mask = 0, need = (uint32_t)n;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int x = tid; x < NWV * 256; x += SNT) (&hist[0][0])[x] = 0;
        __syncthreads();
        for (int i = tid; i < N; i += SNT) {
            const uint32_t u = e[i];
            if ((u & mask) == prefix) atomicAdd(&hist[wv][(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t c = 0;
            for (int x = 0; x < NWV; ++x) c += hist[x][tid];
            total[tid] = c;
        }
        __syncthreads();
        if (tid == 0) {
            // digit d: the tokens above it (acc) number fewer than need, with it at least need
            uint32_t acc = 0;
            int d = 255;
            for (; d > 0; --d) {
                if (acc + total[d] >= need) break;
                acc += total[d];
            }
            sh_prefix = prefix | ((uint32_t)d << shift);
            sh_need = need - acc;
        }
        __syncthreads();
        prefix = sh_prefix;
        need = sh_need;
        mask |= 255u << shift;
    }
    const uint32_t T = prefix;

    int pos = 0, eq_seen = 0;                               // both uniform over the block
    for (int c0 = 0; c0 < N; c0 += SNT) {
        const int i = c0 + tid;
        const uint32_t u = i < N ? e[i] : 0u;
        const bool gt = i < N && u > T, eq = i < N && u == T;
        const uint64_t below = (1ull << lane) - 1ull;       // lanes before this one
        const uint64_t beq = __ballot(eq);
        if (lane == 0) wave_eq[wv] = __popcll(beq);
        __syncthreads();
        int eq_rank = eq_seen + __popcll(beq & below), eq_tot = 0;
        for (int x = 0; x < NWV; ++x) {
            if (x < wv) eq_rank += wave_eq[x];
            eq_tot += wave_eq[x];
        }
        const bool take = gt || (eq && eq_rank < (int)need);
        const uint64_t bt = __ballot(take);
        if (lane == 0) wave_take[wv] = __popcll(bt);
        __syncthreads();
        int at = pos + __popcll(bt & below), tot = 0;
        for (int x = 0; x < NWV; ++x) {
            if (x < wv) at += wave_take[x];
            tot += wave_take[x];
        }
        if (take) out[at] = i;
        pos += tot;
        eq_seen += eq_tot;
        __syncthreads();                                    // wave_* reused next chunk
    }
}

// Token repair: the V^T codes of the repaired keys, gathered once per (b, h) (blockIdx.x)
// into [D][ldr] (ldr = n rounded up to 64, zero padded) for the forward's key correction.
// grid (B*H, D / 8).
__global__ __launch_bounds__(NT) void gather_v_repair_kernel(const uint8_t* __restrict__ v8t,
                                                            int64_t ldv, int D,
                                                            const int32_t* __restrict__ k_sel,
                                                            int n, int ldr,
                                                            uint8_t* __restrict__ out) {
    // blockIdx.y: a group of 8 channels
    const int bh = blockIdx.x, c0 = blockIdx.y * 8;
    const uint8_t* src = v8t + (int64_t)bh * D * ldv;
    const int32_t* sel = k_sel + (int64_t)bh * n;
    uint8_t* dst = out + (int64_t)bh * D * ldr;
    for (int i = threadIdx.x; i < 8 * ldr; i += NT) {
        const int c = c0 + i / ldr, r = i % ldr;
        dst[(int64_t)c * ldr + r] = r < n ? src[(int64_t)c * ldv + sel[r]] : (uint8_t)0;
    }
}

template <int D, bool GATHER>
hipError_t launch_d(const void* q, const void* k, const void* vt, const StreamTable& st, int B,
                    int H, int N, int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                    float* q_scale, float* k_scale, float* v_scale, void* q_hi, void* k_hi,
                    int32_t* hi_idx, float* ch_amax, hipStream_t stream) {
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    if (mode == 1) {
        const int n_amax = B * H * 2 * D;
        hipLaunchKernelGGL(clear_kernel, dim3((n_amax + NT - 1) / NT), dim3(NT), 0, stream,
                           ch_amax, n_amax);
        hipLaunchKernelGGL((chan_amax_kernel<D, GATHER>), dim3(nblk, B * H, 2), dim3(NT), 0,
                           stream, qq, kk, st, H, N, ch_amax);
        hipLaunchKernelGGL(select_hi_kernel<D>, dim3(B * H), dim3(64), 0, stream, ch_amax,
                           hi_idx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((quant_qk_kernel<D, true, GATHER>), dim3(nblk, B * H, 2), dim3(NT), 0,
                           stream, qq, kk, st, H, N, static_cast<uint8_t*>(q8),
                           static_cast<uint8_t*>(k8), q_scale, k_scale, nblk, hi_idx,
                           static_cast<uint16_t*>(q_hi), static_cast<uint16_t*>(k_hi));
    } else {
        hipLaunchKernelGGL((quant_qk_kernel<D, false, GATHER>), dim3(nblk, B * H, 2), dim3(NT),
                           0, stream, qq, kk, st, H, N, static_cast<uint8_t*>(q8),
                           static_cast<uint8_t*>(k8), q_scale, k_scale, nblk, nullptr, nullptr,
                           nullptr);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (GATHER) {
        const int n_vs = B * H * D;
        hipLaunchKernelGGL(clear_kernel, dim3((n_vs + NT - 1) / NT), dim3(NT), 0, stream,
                           v_scale, n_vs);
        hipLaunchKernelGGL(v_amax_kernel<D>, dim3((N + 255) / 256, B * H), dim3(NT), 0, stream,
                           st, H, N, v_scale);
        hipLaunchKernelGGL(quant_vt_kernel<D>, dim3((int)((ldv + 63) / 64), B * H), dim3(NT), 0,
                           stream, st, H, N, ldv, v_scale, static_cast<uint8_t*>(v8t));
        hipLaunchKernelGGL(v_scale_final_kernel, dim3((n_vs + NT - 1) / NT), dim3(NT), 0,
                           stream, v_scale, n_vs);
    } else {
        hipLaunchKernelGGL(quant_v_kernel, dim3(D, B * H), dim3(NT), 0, stream,
                           static_cast<const uint16_t*>(vt), N, D, ldv,
                           static_cast<uint8_t*>(v8t), v_scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const void* q, const void* k, const void* vt, int B, int H, int N,
                            int D, int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                            float* q_scale, float* k_scale, float* v_scale, void* q_hi,
                            void* k_hi, int32_t* hi_idx, float* ch_amax, hipStream_t stream) {
    const StreamTable none{};
    return D == 64 ? launch_d<64, false>(q, k, vt, none, B, H, N, ldv, mode, q8, k8, v8t,
                                         q_scale, k_scale, v_scale, q_hi, k_hi, hi_idx, ch_amax,
                                         stream)
                   : launch_d<128, false>(q, k, vt, none, B, H, N, ldv, mode, q8, k8, v8t,
                                          q_scale, k_scale, v_scale, q_hi, k_hi, hi_idx, ch_amax,
                                          stream);
}

hipError_t launch_quant_fp8_repair(const void* q, const void* k, const void* vt, int B, int H,
                                   int N, int D, int64_t ldv, int n_repair, void* q8, void* k8,
                                   void* v8t, float* q_scale, float* k_scale, float* v_scale,
                                   float* q_err, float* k_err, int32_t* q_sel, int32_t* k_sel,
                                   void* v8t_sel, hipStream_t stream) {
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;
    const uint16_t* qq = static_cast<const uint16_t*>(q);
    const uint16_t* kk = static_cast<const uint16_t*>(k);
    const StreamTable none{};
    if (D == 64)
        hipLaunchKernelGGL((quant_qk_kernel<64, false, false, true>), dim3(nblk, B * H, 2),
                           dim3(NT), 0, stream, qq, kk, none, H, N, static_cast<uint8_t*>(q8),
                           static_cast<uint8_t*>(k8), q_scale, k_scale, nblk, nullptr, nullptr,
                           nullptr, q_err, k_err);
    else
        hipLaunchKernelGGL((quant_qk_kernel<128, false, false, true>), dim3(nblk, B * H, 2),
                           dim3(NT), 0, stream, qq, kk, none, H, N, static_cast<uint8_t*>(q8),
                           static_cast<uint8_t*>(k8), q_scale, k_scale, nblk, nullptr, nullptr,
                           nullptr, q_err, k_err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quant_v_kernel, dim3(D, B * H), dim3(NT), 0, stream,
                       static_cast<const uint16_t*>(vt), N, D, ldv, static_cast<uint8_t*>(v8t),
                       v_scale);
    if (n_repair > 0) {
        hipLaunchKernelGGL(select_repair_kernel, dim3(B * H, 2), dim3(SNT), 0, stream, q_err,
                           k_err, N, n_repair, q_sel, k_sel);
        hipLaunchKernelGGL(gather_v_repair_kernel, dim3(B * H, D / 8), dim3(NT), 0, stream,
                           static_cast<const uint8_t*>(v8t), ldv, D, k_sel, n_repair,
                           (n_repair + 63) / 64 * 64, static_cast<uint8_t*>(v8t_sel));
    }
    return hipGetLastError();
}

hipError_t launch_quant_fp8_streams(const StreamTable& st, int B, int H, int N, int D,
                                    int64_t ldv, int mode, void* q8, void* k8, void* v8t,
                                    float* q_scale, float* k_scale, float* v_scale, void* q_hi,
                                    void* k_hi, int32_t* hi_idx, float* ch_amax,
                                    hipStream_t stream) {
    return D == 64 ? launch_d<64, true>(nullptr, nullptr, nullptr, st, B, H, N, ldv, mode, q8, k8,
                                        v8t, q_scale, k_scale, v_scale, q_hi, k_hi, hi_idx,
                                        ch_amax, stream)
                   : launch_d<128, true>(nullptr, nullptr, nullptr, st, B, H, N, ldv, mode, q8,
                                         k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi, hi_idx,
                                         ch_amax, stream);
}

}  // namespace ja

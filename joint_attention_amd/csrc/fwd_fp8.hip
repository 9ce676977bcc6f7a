// Joint attention forward on fp8 (OCP E4M3) operands (gfx950).
//
// The fp8 attention variant of the VisualGen FLUX 3 article (everytik.com translation,
// section 量化注意力与稀疏注意力: fp8 Q/K and fp8 V), on the codes and scales that
// quant_fp8 produces.  Same work split and operand mapping as the bf16 kernel (S^T =
// K Q^T with one query per lane, O^T = V^T P^T with P^T taken from the score
// registers), on v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3).
//
// Work split.  One workgroup = NW waves of 32 query rows (256 rows for D = 128); keys
// come in tiles of 64, one k-depth of the fp8 P V product.  A wave's 32 rows lie inside
// one 128-row Q scale block and a 64-key tile inside one K scale block, so
// scale * qs * ks * log2(e) is one factor per (lane, tile), applied in the FMA that
// subtracts the running maximum.
//
// Software pipeline (as in the bf16 kernel).  Iteration j runs the softmax of tile j on
// the vector ALU while the matrix cores run P(j-1) V(j-1) and Q K(j+1)^T, written as an
// explicit sequence of steps (operand reads a few steps ahead, one MFMA and a slice of
// the softmax each) separated by scheduling fences.  K, V^T (and the kept channels of
// the split mode) are staged in registers one iteration ahead and double-buffered in
// LDS, with one barrier per iteration.  LDS rows are XOR-swizzled so that each LDS
// access is conflict-free on gfx950: a read serves 256 bytes per clock (16 lanes of a
// 16-byte read, 32 of an 8-byte one), a write 128 bytes (8 lanes of a 16-byte write), and
// the lanes served together must hit distinct 4-byte banks of that window.
//
// Softmax.  The running maximum M is an integer (base 2), raised only when some score
// of the tile exceeds it by more than 0.75 (a wave-uniform ballot; the two wave halves
// are combined and O rescaled only then), and then to one above the tile's integer
// maximum.  Every rescale is an exact power of two, and above e4m3's subnormal range P's
// rounding depends neither on M nor on the order keys arrive in.  P is stored as
// e4m3(2^8 * 2^(t - M)), below 2^8.75, with the 2^8 folded into the exponent; the row
// sum takes the same unrounded fp32 numerators and the 2^8 cancels in O = acc / l.  The
// per-channel V scale is applied in the epilogue.
//
// Split mode (HI): the 16 kept channels of Q and K (bf16, already divided by their
// power-of-two block scales) add one v_mfma_f32_32x32x16_bf16 per 32x32 score block
// into the same accumulator, so t = (q8.k8 + q_hi.k_hi) * qs * ks * scale * log2 e.
// Token repair (the repair budget of VC-Attention FP8, same article section): the listed
// queries and keys enter the logits with their exact bf16 values.  The main kernel above
// runs unchanged on the codes and writes O and lse; fwd_fp8_keyfix_kernel then replaces,
// in every row, each listed key's code term by its exact-value term: with the row's
// total L = e^lse it adds (e4m3(2^(8 + t~ - M')) - e4m3(2^(8 + t^ - M'))) 2^(M' - 8) v
// to L O and 2^t~ - 2^t^ to L, for an integer M' (shifting by an integer power of two
// leaves e4m3 rounding unchanged while the value stays above the subnormal range, so
// the loop's code term cancels exactly for every key whose weight is within 2^-12 of
// the row maximum's, the loop's M being at most two above that maximum).  Workgroups appended to the main grid
// (repair_rows) recompute the listed query rows from their exact values; the main and the
// correction kernels leave those rows alone.
#include <type_traits>

#include "ja_device.h"
#include "ja_launch.h"
#include "splitkv_merge.h"

namespace ja {
namespace {

#ifndef FP8_LEAD
#define FP8_LEAD 2          // operand reads this many MFMA steps ahead
#endif
#ifndef FP8_NW128
#define FP8_NW128 8
#endif
// the running maximum M rises only when some logit exceeds it by more than FP8_GROW_SLACK
// (P = e4m3(2^(8 + t - M)) then stays below 2^8.75 < 448), and then to FP8_GROW_HEADROOM
// above the tile's integer maximum, so that fewer tiles pay for a rescale of O
#ifndef FP8_GROW_SLACK
#define FP8_GROW_SLACK 0.75f
#endif
#ifndef FP8_GROW_HEADROOM
#define FP8_GROW_HEADROOM 1.f
#endif

__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// 8 e4m3 codes (two words, bytes in channel order) -> 8 bf16, exact
__device__ inline bf16x8 e4m3x8_to_bf16(int w0, int w1) {
    bf16x8 r;
    const floatx2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
    const floatx2 b2 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
    const floatx2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
    const floatx2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
    r[0] = (__bf16)a[0];
    r[1] = (__bf16)a[1];
    r[2] = (__bf16)b2[0];
    r[3] = (__bf16)b2[1];
    r[4] = (__bf16)c[0];
    r[5] = (__bf16)c[1];
    r[6] = (__bf16)d[0];
    r[7] = (__bf16)d[1];
    return r;
}

// channel of element e (0..7) of k-step c16 of a bf16 product over the head's channels
// for lane half hh: the 8 channels a lane half holds per k-step are the ones the fp8
// Q operand already holds in that lane (64 (c16 / 4) + 32 hh + 8 (c16 % 4) + e)
__device__ inline int rep_channel(int c16, int hh) { return 64 * (c16 / 4) + 32 * hh + 8 * (c16 % 4); }

// Token repair, the listed query rows: the workgroups after the main grid of
// fwd_fp8_kernel<..., RROWS> (dispatched last, they fill the CUs its last round leaves
// idle), block rb of (b, h) slice bh.  The 32 rows of a workgroup (lane r32 <-> row
// QSEL[32 rb + r32]) take their exact bf16 Q
// values; keys are the codes widened to bf16 (exact), or for listed keys their exact
// values divided by the block scale (exact: a power of two), so that one factor
// c2 * k_scale per tile again turns products into base-2 logits.  Wave w visits tiles
// w, w + NWR, .., with the next tile's K codes loaded into registers while the
// current one is computed; P (e4m3, integer running maximum as in the main kernel)
// times V^T codes runs on the fp8 matrix cores.  The waves' states (all maxima are
// integers, so every rescale is a power of two) are merged through LDS in wave order.
template <int D, int NWR>
__device__ __forceinline__ void repair_rows(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const uint8_t* __restrict__ K8,
    const uint8_t* __restrict__ V8T, const float* __restrict__ KS, const float* __restrict__ VS,
    const int32_t* __restrict__ QSEL, const int32_t* __restrict__ KSEL, int NREP, int H, int N,
    int64_t ldv, float c2, __bf16* __restrict__ O, float* __restrict__ LSE, const int rb,
    const int bh) {
    constexpr int NT = NWR * 64, BC = 64, KB = BC / 32, NOB = D / 32, NK16 = D / 16;
    __shared__ uint32_t kmask[JA_REPAIR_MAX_N / 32];
    __shared__ float sm[NWR][32], sl[NWR][32];
    __shared__ float so[D][33];                        // [channel][row], padded
    __shared__ __attribute__((aligned(16))) __bf16 sq[32][D + 8];   // exact Q rows, padded
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, hh = lane >> 5;
    const int b = bh / H, h = bh - b * H;
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;

    // listed keys as a bitmask; the merge buffer starts at zero
    const int nwords = (N + 31) / 32;
    for (int i = tid; i < nwords; i += NT) kmask[i] = 0;
    for (int i = tid; i < D * 33; i += NT) (&so[0][0])[i] = 0.f;
    __syncthreads();
    // list entries are clamped to [0, N): a caller's bad list gives wrong rows, never an
    // access outside Q, K, O, LSE or the LDS mask
    for (int i = tid; i < NREP; i += NT) {
        const int key = min(max(KSEL[(int64_t)bh * NREP + i], 0), N - 1);
        atomicOr(&kmask[key >> 5], 1u << (key & 31));
    }
    __syncthreads();

    const int slot = rb * 32 + r32;
    const int qi = min(max(QSEL[(int64_t)bh * NREP + min(slot, NREP - 1)], 0), N - 1);
    for (int x = tid; x < 32 * (D / 8); x += NT) {     // the 32 rows' exact Q -> LDS
        const int r = x / (D / 8), u = x % (D / 8);
        const int qr = min(max(QSEL[(int64_t)bh * NREP + min(rb * 32 + r, NREP - 1)], 0), N - 1);
        *reinterpret_cast<uint4*>(&sq[r][u * 8]) =
            *reinterpret_cast<const uint4*>(Q + ((int64_t)bh * N + qr) * D + u * 8);
    }
    __syncthreads();
    auto q_op = [&](int c16) {                          // B operand: this lane's row
        return *reinterpret_cast<const bf16x8*>(&sq[r32][rep_channel(c16, hh)]);
    };
    const uint8_t* K8bh = K8 + (int64_t)bh * N * D;
    const __bf16* Kbh = K + (int64_t)bh * N * D;
    const uint8_t* Vbh = V8T + (int64_t)bh * D * ldv;

    // a tile's K codes (row kb*32 + swap_bits23(r32), 8 channels per k-step) and V^T
    // codes (row 32 i + r32, keys 16 u + 8 hh ..)
    // (the k-steps c16 = 2x, 2x + 1 of a lane are 16 consecutive channels: one load)
    auto load_k = [&](int t, uint2 (&kx)[KB][NK16]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int key = min(t * BC + kb * 32 + swap_bits23(r32), N - 1);
#pragma unroll
            for (int c16 = 0; c16 < NK16; c16 += 2) {
                const uint4 x = *reinterpret_cast<const uint4*>(K8bh + (int64_t)key * D +
                                                                rep_channel(c16, hh));
                kx[kb][c16] = make_uint2(x.x, x.y);
                kx[kb][c16 + 1] = make_uint2(x.z, x.w);
            }
        }
    };
    auto load_v = [&](int t, uint2 (&vx)[NOB][4]) {
#pragma unroll
        for (int i = 0; i < NOB; ++i) {
            const uint8_t* vrow = Vbh + (int64_t)(32 * i + r32) * ldv;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k0 = t * BC + 16 * u + 8 * hh;
                uint2 x = make_uint2(0, 0);
                if (k0 < N) {
                    // k0 < N, k0 % 8 == 0 and ldv % 16 == 0 keep the 8 bytes in the row
                    x = *reinterpret_cast<const uint2*>(vrow + k0);
                    if (k0 + 8 > N) {
                        const int keep = N - k0;              // 1..7 bytes
                        const uint64_t mk = (1ull << (8 * keep)) - 1ull;
                        const uint64_t v64 = (((uint64_t)x.y << 32) | x.x) & mk;
                        x = make_uint2((uint32_t)v64, (uint32_t)(v64 >> 32));
                    }
                }
                vx[i][u] = x;
            }
        }
    };
    uint2 kc[KB][NK16];

    floatx16 oacc[NOB];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int a = 0; a < 16; ++a) oacc[ob][a] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int nkt = (N + BC - 1) / BC;
    if (w < nkt) load_k(w, kc);
    for (int t = w; t < nkt; t += NWR) {
        uint2 vc[NOB][4], kn[KB][NK16];
        load_v(t, vc);                                // in flight during QK and the softmax
        if (t + NWR < nkt) load_k(t + NWR, kn);
        const float ks = KS[(int64_t)bh * nblk + (t * BC) / JA_QK_BLOCK];
        const float inv_ks = 1.f / ks;                // a power of two: exact
        floatx16 s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int key = min(t * BC + kb * 32 + swap_bits23(r32), N - 1);
            const bool rep = (kmask[key >> 5] >> (key & 31)) & 1u;
#pragma unroll
            for (int a = 0; a < 16; ++a) s[kb][a] = 0.f;
            if (__ballot(rep) == 0) {                 // no listed key in this block
#pragma unroll
                for (int c16 = 0; c16 < NK16; ++c16)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        e4m3x8_to_bf16((int)kc[kb][c16].x, (int)kc[kb][c16].y), q_op(c16), s[kb],
                        0, 0, 0);
            } else {
#pragma unroll
                for (int c16 = 0; c16 < NK16; ++c16) {
                    bf16x8 ak = e4m3x8_to_bf16((int)kc[kb][c16].x, (int)kc[kb][c16].y);
                    if (rep) {
                        const bf16x8 x = *reinterpret_cast<const bf16x8*>(
                            Kbh + (int64_t)key * D + rep_channel(c16, hh));
#pragma unroll
                        for (int e = 0; e < 8; ++e) ak[e] = (__bf16)((float)x[e] * inv_ks);
                    }
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, q_op(c16), s[kb], 0, 0, 0);
                }
            }
        }
        const float f = c2 * ks;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int key = t * BC + kb * 32 + 16 * (a / 8) + 8 * hh + (a % 8);
                if (key >= N) s[kb][a] = -INFINITY;
                mx = fmaxf(mx, s[kb][a]);
            }
        const float tmax = mx * f;
        if (__ballot(tmax > m) != 0) {
            const float m_new = fmaxf(m, ceilf(wave_halves_max(tmax)));
            const float alpha = (m == -INFINITY) ? 0.f : ldexpf(1.f, (int)(m - m_new));
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int a = 0; a < 16; ++a) oacc[ob][a] *= alpha;
        }
        const float bias = 8.f - m;
        intx8 pf;
#pragma unroll
        for (int k = 0; k < 4 * KB; ++k) {
            const int kb = k / 4, d = k % 4;
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[kb][4 * d + e], f, bias));
            l += (p[0] + p[1]) + (p[2] + p[3]);
            const int wp = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            pf[k] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wp, true);
        }
#pragma unroll
        for (int i = 0; i < NOB; ++i) {
            intx8 av;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                av[2 * u] = (int)vc[i][u].x;
                av[2 * u + 1] = (int)vc[i][u].y;
            }
            oacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pf, oacc[i], 0, 0, 0, 0,
                                                                     0, 0);
        }
        if (t + NWR < nkt) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int c16 = 0; c16 < NK16; ++c16) kc[kb][c16] = kn[kb][c16];
        }
    }

    // merge the waves: rows' maxima, then the rescaled numerators added in wave order
    const float lw = wave_halves_sum(l);
    if (hh == 0) {
        sm[w][r32] = m;
        sl[w][r32] = lw;
    }
    __syncthreads();
    float mt = sm[0][r32];
#pragma unroll
    for (int x = 1; x < NWR; ++x) mt = fmaxf(mt, sm[x][r32]);
    const float sc = (m == -INFINITY) ? 0.f : ldexpf(1.f, (int)(m - mt));
    // O^T slot (ob, a): channel ob*32 + 8 (a / 4) + 4 hh + a % 4, row r32
    for (int x = 0; x < NWR; ++x) {
        if (w == x) {
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int a = 0; a < 16; ++a)
                    so[ob * 32 + 8 * (a / 4) + 4 * hh + (a % 4)][r32] += oacc[ob][a] * sc;
        }
        __syncthreads();
    }
    if (w == 0 && slot < NREP) {
        float lt = 0.f;
#pragma unroll
        for (int x = 0; x < NWR; ++x)
            lt += sm[x][r32] == -INFINITY ? 0.f : sl[x][r32] * ldexpf(1.f, (int)(sm[x][r32] - mt));
        const float inv = 1.f / lt;
        __bf16* orow = O + (((int64_t)b * N + qi) * H + h) * D;
        const float* vs = VS + (int64_t)bh * D;
        for (int c = hh; c < D; c += 2) orow[c] = (__bf16)(so[c][r32] * inv * vs[c]);
        if (hh == 0) LSE[(int64_t)bh * N + qi] = (mt - 8.f + log2f(lt)) * kLn2;
    }
}

// RROWS (token repair): workgroups past `total` recompute the listed query rows
// (repair_rows); the main workgroups leave those rows to them.
// PARTIAL (split-KV): the query tiles from n_full on (the last, partial round of
// workgroups) run as n_split key ranges of whole tiles, each writing its normalised fp32
// output (V scale applied) and natural-log lse for splitkv_merge_kernel.
template <int D, int NW, bool HI, bool RROWS = false, bool PARTIAL = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8T,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    const __bf16* __restrict__ QH, const __bf16* __restrict__ KH,
    int H, int N, int64_t ldv, float c2, __bf16* __restrict__ O, float* __restrict__ LSE,
    int n_qtiles, int total, const __bf16* __restrict__ QX = nullptr,
    const __bf16* __restrict__ KX = nullptr, const int32_t* __restrict__ QSEL = nullptr,
    const int32_t* __restrict__ KSEL = nullptr, int NREP = 0, int n_split = 1,
    float* __restrict__ OP = nullptr, float* __restrict__ LP = nullptr, int n_full = 0) {
    static_assert(!(HI && RROWS), "token repair runs on the plain codes");
    static_assert(!(RROWS && PARTIAL), "one variant at a time");
    if constexpr (RROWS) {
        if ((int)blockIdx.x >= total) {
            const int r = (int)blockIdx.x - total, nb = (NREP + 31) / 32;
            repair_rows<D, NW>(QX, KX, K8, V8T, KS, VS, QSEL, KSEL, NREP, H, N, ldv, c2, O, LSE,
                               r % nb, r / nb);
            return;
        }
    }
    constexpr int NTHREADS = NW * 64;
    constexpr int BR = NW * 32;              // query rows per workgroup
    constexpr int BC = 64;                   // keys per tile
    constexpr int KB = BC / 32;              // 32-key score blocks per tile
    constexpr int KROWB = D;                 // bytes per K row
    constexpr int DC = D / 16;               // 16-byte chunks per K row
    constexpr int KRPB = 256 / KROWB;        // K rows per 256-byte line of the 64 LDS banks
    constexpr int NQC = D / 64;              // k-steps of the QK product (64 channels each)
    constexpr int NOB = D / 32;              // 32-channel output blocks
    constexpr int VCPR = BC / 16;            // 16-byte chunks per V^T row
    constexpr int HC = JA_HI_CHANNELS;       // kept channels (bf16), 2 x 16 bytes per key
    constexpr int KCH = BC * DC / NTHREADS;  // 16-byte K chunks per thread and tile
    constexpr int VCH = D * (BC / 16) / NTHREADS;
    static_assert(KCH >= 1 && VCH >= 1 && KCH * NTHREADS == BC * DC &&
                  VCH * NTHREADS == D * (BC / 16) && NTHREADS >= 2 * BC, "chunk mapping");
    static_assert(JA_QK_BLOCK % 32 == 0 && JA_QK_BLOCK % BC == 0,
                  "a wave's rows and a key tile must each lie in one scale block");
    __shared__ __attribute__((aligned(16))) uint8_t sk[2][BC * KROWB];
    __shared__ __attribute__((aligned(16))) uint8_t sv[2][D * BC];
    __shared__ __attribute__((aligned(16))) __bf16 skh[2][HI ? BC * HC : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, hh = lane >> 5;
    // PARTIAL: the whole-round workgroups and the split ones are renumbered separately, so
    // that both spread evenly over the XCDs (n_full is a multiple of the slot count)
    const int bid = blockIdx.x;
    const int wg = !PARTIAL ? xcd_remap(bid, total)
                   : bid < n_full ? xcd_remap(bid, n_full)
                                  : n_full + xcd_remap(bid - n_full, total - n_full);
    int unit = wg, split = 0;
    bool part_wg = false;
    if constexpr (PARTIAL) {
        if (wg >= n_full) {
            const int x = wg - n_full;
            unit = n_full + x / n_split;
            split = x - (x / n_split) * n_split;
            part_wg = true;
        }
    }
    const int bh = unit / n_qtiles, qt = unit - bh * n_qtiles;
    const int b = bh / H, h = bh - b * H;
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;
    const uint8_t* Qbh = Q8 + (int64_t)bh * N * D;
    const uint8_t* Kbh = K8 + (int64_t)bh * N * D;
    const uint8_t* Vbh = V8T + (int64_t)bh * D * ldv;
    const __bf16* KHbh = HI ? KH + (int64_t)bh * N * HC : nullptr;
    const float* KSbh = KS + (int64_t)bh * nblk;
    int nkt = (N + BC - 1) / BC;
    int t_begin = 0;                               // PARTIAL: first key tile of the range
    if (PARTIAL && part_wg) {
        // n_split <= the number of key tiles (the launcher clamps it): no range is empty
        const int all = nkt;
        t_begin = (int)((int64_t)split * all / n_split);
        nkt = (int)((int64_t)(split + 1) * all / n_split) - t_begin;
    }
    // keys of this workgroup: [t_begin * BC, kend).  A range of one tile runs as two, the
    // second masked out entirely (its P is exactly zero), so that every workgroup takes the
    // one pipelined path (a separate one-tile path kept values live across both and made
    // the compiler spill them)
    const int kend = min(N, (t_begin + nkt) * BC);
    nkt = max(nkt, 2);
    // RROWS: which of this workgroup's rows are listed (left to the row recomputation)
    __shared__ uint32_t rmask[RROWS ? NW : 1];
    if constexpr (RROWS) {
        if (tid < NW) rmask[tid] = 0;
        __syncthreads();
        const int r0 = qt * BR;
        for (int i = tid; i < NREP; i += NTHREADS) {
            const int r = QSEL[(int64_t)bh * NREP + i] - r0;
            if (r >= 0 && r < BR) atomicOr(&rmask[r >> 5], 1u << (r & 31));
        }
        __syncthreads();
    }

    // ---- staging: chunk x = tid + i * NTHREADS of a tile is K row x / DC, 16-byte
    //      chunk x % DC, and V^T row x / 4, keys 16 (x % 4) .. + 15; threads t < 128
    //      also own half a kept-channel row
    uint4 kst[KCH], vst[VCH], hst = make_uint4(0, 0, 0, 0);
    // V^T in LDS: chunk c = 2 hh + jj of row vr holds the keys that lane half hh feeds
    // to the PV product as its 16-byte piece jj, keys 32 jj + 8 hh + (0..7) and 32 jj +
    // 16 + 8 hh + (0..7), so an operand is two 16-byte reads; it sits at chunk
    // c ^ vswz(vr).  The 16 lanes of such a read (16 rows, four per 256-byte bank line)
    // then meet four distinct swizzles, and the 16 lanes of an 8-byte staging write (rows
    // vr .. vr + 3 in a 128-byte window) put rows vr and vr + 2 in different chunks.
    auto vswz = [](int r) { return ((r / 4) % VCPR) ^ (((r / 2) & 1) << 1); };
    auto load_k = [&](int kt) {
        const int k0 = (t_begin + kt) * BC;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int x = tid + i * NTHREADS, kr = x / DC, kc = x % DC;
            const int key = min(k0 + kr, N - 1);        // rows past N: any finite row
            kst[i] = *reinterpret_cast<const uint4*>(Kbh + (int64_t)key * D + kc * 16);
        }
        if (HI && tid < 2 * BC) {
            const int hkey = k0 + tid / 2;
            hst = make_uint4(0, 0, 0, 0);
            if (hkey < N)
                hst = *reinterpret_cast<const uint4*>(KHbh + (int64_t)hkey * HC + (tid % 2) * 8);
        }
    };
    // 8 bytes of V^T row vr from key `key` (a multiple of 8): keys at or past N read as zero
    auto v_piece = [&](int vr, int key) {
        uint2 piece = make_uint2(0, 0);
        if (key < N) {
            // key < N, key % 8 == 0 and ldv % 16 == 0 keep the 8 bytes in the row
            const uint2 v = *reinterpret_cast<const uint2*>(Vbh + (int64_t)vr * ldv + key);
            uint32_t wv[2] = {v.x, v.y};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (key + e >= N) wv[e / 4] &= ~(0xFFu << (8 * (e % 4)));
            piece = make_uint2(wv[0], wv[1]);
        }
        return piece;
    };
    auto load_v = [&](int kt) {
        const int k0 = (t_begin + kt) * BC;
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int x = tid + i * NTHREADS, vr = x / VCPR, c = x % VCPR;
            // keys 16 c .. 16 c + 15: the pieces of chunks (jj = c / 2, hh = 0 and 1)
            const int key0 = k0 + 16 * c;
            uint2 p0, p1;
            if (key0 + 16 <= N) {
                const uint4 v = *reinterpret_cast<const uint4*>(Vbh + (int64_t)vr * ldv + key0);
                p0 = make_uint2(v.x, v.y);
                p1 = make_uint2(v.z, v.w);
            } else {
                p0 = v_piece(vr, key0);
                p1 = v_piece(vr, key0 + 8);
            }
            vst[i] = make_uint4(p0.x, p0.y, p1.x, p1.y);
        }
    };
    auto store_k = [&](int slot) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int x = tid + i * NTHREADS, kr = x / DC, kc = x % DC;
            *reinterpret_cast<uint4*>(&sk[slot][kr * KROWB + ((kc ^ ((kr / KRPB) % DC)) * 16)]) =
                kst[i];
        }
        if (HI && tid < 2 * BC) {
            const int row = tid / 2, half = (tid % 2) ^ ((row >> 3) & 1);
            *reinterpret_cast<uint4*>(&skh[slot][row * HC + half * 8]) = hst;
        }
    };
    auto store_v = [&](int slot) {
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int x = tid + i * NTHREADS, vr = x / VCPR, c = x % VCPR;
            // keys 16 c ..: half 0 -> chunk (hh 0, jj c / 2), half 1 -> chunk (hh 1, jj c / 2),
            // each at byte 8 (c % 2) of the chunk
            uint8_t* row = &sv[slot][vr * BC + 8 * (c % 2)];
            *reinterpret_cast<uint2*>(row + ((c / 2) ^ vswz(vr)) * 16) = make_uint2(vst[i].x, vst[i].y);
            *reinterpret_cast<uint2*>(row + ((2 + c / 2) ^ vswz(vr)) * 16) =
                make_uint2(vst[i].z, vst[i].w);
        }
    };

    // ---- resident state
    const int q_row = qt * BR + w * 32 + r32;
    const int q_ld = min(q_row, N - 1);
    // all rows of a wave (clamped ones included) share one Q scale block
    const float qsc2 = QS[(int64_t)bh * nblk + q_ld / JA_QK_BLOCK] * c2;
    intx8 qf[NQC];
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
        const uint4* p = reinterpret_cast<const uint4*>(Qbh + (int64_t)q_ld * D + 64 * c + 32 * hh);
        const uint4 x0 = p[0], x1 = p[1];
        qf[c] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
    bf16x8 qhf = {};
    if (HI) qhf = *reinterpret_cast<const bf16x8*>(QH + ((int64_t)bh * N + q_ld) * HC + 8 * hh);
    floatx16 oacc[NOB];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int a = 0; a < 16; ++a) oacc[ob][a] = 0.f;
    float m = -INFINITY, l = 0.f;                 // integer running max (base 2); row sum

    // ---- MFMA steps.  PV step i (< NOB): A = V^T rows 32 i.. (64 keys), B = P^T.
    //      QK step i (< NQK): c = i / KB, kb = i % KB: A = K rows kb*32.. (bits 2/3
    //      swapped), channels 64c..; B = Q.  HI step i (< KB): A = kept channels of
    //      K rows kb*32.., B = kept channels of Q.
    constexpr int NPV = NOB;
    constexpr int NQK = NQC * KB;
    constexpr int NHI = HI ? KB : 0;
    constexpr int NQ = NQK + NHI;
    auto pv_operand = [&](int slot, int i) {
        // lane half hh: keys {16 u + 8 hh + (0..7)}, u = 0..3, as chunks 2 hh and 2 hh + 1
        const int vrow = i * 32 + r32, z = vswz(vrow);
        const uint4 x0 = *reinterpret_cast<const uint4*>(&sv[slot][vrow * BC + (((2 * hh) ^ z) * 16)]);
        const uint4 x1 =
            *reinterpret_cast<const uint4*>(&sv[slot][vrow * BC + (((2 * hh + 1) ^ z) * 16)]);
        return intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    };
    auto q_operand = [&](int slot, int i) {
        intx8 av;
        if (i < NQK) {
            const int c = i / KB, kb = i % KB;
            const int krow = kb * 32 + swap_bits23(r32);
            const int kz = (krow / KRPB) % DC;
            const int u0 = 4 * c + 2 * hh;            // channels 64c + 32hh .. +31
            const uint4 x0 = *reinterpret_cast<const uint4*>(&sk[slot][krow * KROWB + ((u0 ^ kz) * 16)]);
            const uint4 x1 =
                *reinterpret_cast<const uint4*>(&sk[slot][krow * KROWB + (((u0 + 1) ^ kz) * 16)]);
            av = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                       (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        } else {
            const int kb = i - NQK;
            const int krow = kb * 32 + swap_bits23(r32);
            const int half = hh ^ ((krow >> 3) & 1);
            const uint4 x = *reinterpret_cast<const uint4*>(&skh[slot][krow * HC + half * 8]);
            av = intx8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        }
        return av;
    };

    floatx16 sA[KB], sB[KB];                      // score tiles, alternating with parity
    intx8 pA, pB;                                 // P^T tiles (e4m3), alternating

    auto mfma_pv = [&](int i, const intx8& av, const intx8& pf) {
        oacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pf, oacc[i], 0, 0, 0, 0,
                                                                 0, 0);
    };
    auto mfma_q = [&](int i, const intx8& av, floatx16 (&s)[KB]) {
        if (i < NQK) {
            const int c = i / KB, kb = i % KB;
            if (c == 0) {
                const floatx16 zero = {};
                s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qf[c], zero, 0, 0, 0,
                                                                       0, 0, 0);
            } else {
                s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qf[c], s[kb], 0, 0, 0,
                                                                       0, 0, 0);
            }
        } else {
            const int kb = i - NQK;
            const intx4 a4 = {av[0], av[1], av[2], av[3]};
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), qhf,
                                                            s[kb], 0, 0, 0);
        }
    };
    auto pv_all = [&](int slot, const intx8& pf) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) mfma_pv(i, pv_operand(slot, i), pf);
    };
    auto q_all = [&](int slot, floatx16 (&s)[KB]) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) mfma_q(i, q_operand(slot, i), s);
    };

    // numerators of 4 scores: k = 4 kb + d covers slots 4d .. 4d + 3 of block kb, which
    // become word k of the P^T operand (A-operand slot s of the PV product <-> key
    // kb*32 + 16u + 8hh + e for s = 16kb + 8u + e)
    constexpr int NQUAD = KB * 4;
    auto exp_quad = [&](floatx16 (&s)[KB], intx8& pf, int k, float f, float bias, float& sum) {
        const int kb = k / 4, d = k % 4;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[kb][4 * d + e], f, bias));
        sum += (p[0] + p[1]) + (p[2] + p[3]);
        // both halves of the word are written; its old contents only save a move
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pf[k], false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
        asm volatile("" : "+v"(word));            // keep at this point of the schedule
        asm volatile("" : "+v"(sum));
        pf[k] = word;
    };
    auto mask_tail = [&](floatx16 (&s)[KB], int kt) {
        const int k0 = (t_begin + kt) * BC;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int key = k0 + kb * 32 + 16 * (a / 8) + 8 * hh + (a % 8);
                if (key >= kend) s[kb][a] = -INFINITY;
            }
    };

    // prologue: K_0, K_1 -> LDS; S_0; stage K_2 and V_0
    load_k(0);
    store_k(0);
    load_k(1);
    store_k(1);
    __syncthreads();
    q_all(0, sA);
    load_k(min(2, nkt - 1));
    load_v(0);

    // iteration j: softmax(S_j) || P_{j-1} V_{j-1} and Q K_{j+1}^T; loads V_j, K_{j+2}
    auto iteration = [&](int j, auto parity_tag, auto has_pv_tag, auto has_qk_tag) {
        constexpr int P = decltype(parity_tag)::value;
        constexpr bool HAS_PV = decltype(has_pv_tag)::value;
        constexpr bool HAS_QK = decltype(has_qk_tag)::value;
        constexpr int MY = P;                     // slot for K_{j+2} and V_j
        constexpr int RD = 1 - P;                 // slot holding K_{j+1} and V_{j-1}
        floatx16 (&s_in)[KB] = P ? sB : sA;       // S_j
        floatx16 (&s_out)[KB] = P ? sA : sB;      // S_{j+1}
        intx8& p_out = P ? pB : pA;               // P_j
        intx8& p_in = P ? pA : pB;                // P_{j-1}
        // only a range's first tile (when it is also its last) and its last can reach kend
        if ((!HAS_QK || !HAS_PV) && (t_begin + j + 1) * BC > kend) mask_tail(s_in, j);
        __syncthreads();
        if (HAS_QK) store_k(MY);
        store_v(MY);
        if (HAS_QK) load_k(min(j + 3, nkt - 1));
        load_v(min(j + 1, nkt - 1));

        // (the masked-out tile of a one-tile range may start past the last scale block)
        const float f = qsc2 * KSbh[min(((t_begin + j) * BC) / JA_QK_BLOCK, nblk - 1)];
        float bias = 0.f, alpha = 1.f;
        bool grow = false;
        // raise M only if some score of the tile exceeds it (a wave-uniform branch)
        auto check = [&]() {
            float mx = s_in[0][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s_in[kb][a]);
            const float tmax = mx * f;
            grow = __ballot(tmax > m + FP8_GROW_SLACK) != 0;
            if (grow) {
                asm volatile("");
                const float m_new = fmaxf(m, ceilf(wave_halves_max(tmax)) + FP8_GROW_HEADROOM);
                alpha = (m == -INFINITY) ? 0.f : ldexpf(1.f, (int)(m - m_new));
                m = m_new;
                l *= alpha;
            }
            bias = 8.f - m;
        };

        constexpr int S0 = HAS_PV ? 0 : NPV;
        constexpr int S1 = HAS_QK ? NPV + NQ : NPV;
        constexpr int NST = S1 - S0;
        constexpr int LEAD = FP8_LEAD;
        constexpr int FIRST = 1;                  // steps before the numerators start
        // step order: PV and QK steps alternate while both remain
        auto step_id = [&](int k) -> int {
            if constexpr (HAS_PV && HAS_QK) {
                constexpr int PAIRS = NPV < NQ ? NPV : NQ;
                if (k < 2 * PAIRS) return (k & 1) ? NPV + (k >> 1) : (k >> 1);
                return NPV > NQ ? k - PAIRS : NPV + (k - PAIRS);
            }
            return S0 + k;
        };
        auto load_op = [&](int st) -> intx8 {
            return st < NPV ? pv_operand(RD, st) : q_operand(RD, st - NPV);
        };
        static_assert(NST > FIRST, "every iteration has a product to overlap");
        {
            intx8 opnd[LEAD + 1];
#pragma unroll
            for (int k = 0; k < LEAD; ++k) opnd[k] = load_op(step_id(k));
#pragma unroll
            for (int k = 0; k < NST; ++k) {
                const int st = step_id(k);
                if (k + LEAD < NST) opnd[(k + LEAD) % (LEAD + 1)] = load_op(step_id(k + LEAD));
                if (st < NPV) mfma_pv(st, opnd[k % (LEAD + 1)], p_in);
                else mfma_q(st - NPV, opnd[k % (LEAD + 1)], s_out);
                if (k == 0) check();
                if (k >= FIRST) {
                    const int lo = (k - FIRST) * NQUAD / (NST - FIRST);
                    const int hi = (k - FIRST + 1) * NQUAD / (NST - FIRST);
#pragma unroll
                    for (int e = lo; e < hi; ++e) exp_quad(s_in, p_out, e, f, bias, l);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // O holds P_{j-1} V_{j-1} in the old scale: rescale after those products
        if (grow) {
            asm volatile("");
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int a = 0; a < 16; ++a) oacc[ob][a] *= alpha;
        }
    };

    using F = std::false_type;
    using T = std::true_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    {
        iteration(0, P0{}, F{}, T{});
        int j = 1;
        for (; j + 2 <= nkt - 1; j += 2) {
            iteration(j, P1{}, T{}, T{});
            iteration(j + 1, P0{}, T{}, T{});
        }
        if (j < nkt - 1) {
            iteration(j, P1{}, T{}, T{});
            ++j;
        }
        if (j & 1) iteration(j, P1{}, T{}, F{});
        else iteration(j, P0{}, T{}, F{});
    }

    // epilogue: P_last V_last (V_last was stored in the last iteration)
    {
        const int jl = nkt - 1;
        __syncthreads();
        if (jl & 1) pv_all(1, pB);
        else pv_all(0, pA);
    }

    const float l_tot = wave_halves_sum(l);
    const float inv = 1.f / l_tot;
    if (PARTIAL && part_wg) {
        if (q_row < N) {
            const int64_t r = ((int64_t)(unit - n_full) * n_split + split) * BR + (q_row - qt * BR);
            float* orow = OP + r * D;
            const float* vs = VS + (int64_t)bh * D;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c0 = ob * 32 + j * 8 + hh * 4;
                    *reinterpret_cast<floatx4*>(orow + c0) =
                        floatx4{oacc[ob][4 * j] * inv * vs[c0], oacc[ob][4 * j + 1] * inv * vs[c0 + 1],
                                oacc[ob][4 * j + 2] * inv * vs[c0 + 2],
                                oacc[ob][4 * j + 3] * inv * vs[c0 + 3]};
                }
            if (hh == 0) LP[r] = (m - 8.f + log2f(l_tot)) * kLn2;
        }
        return;
    }
    const bool listed = RROWS && ((rmask[w] >> r32) & 1u);
    if (q_row < N && !listed) {
        __bf16* orow = O + (((int64_t)b * N + q_row) * H + h) * D;
        const float* vs = VS + (int64_t)bh * D;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c0 = ob * 32 + j * 8 + hh * 4;
                // v_scale is only 4-byte aligned by contract: four scalar loads
                floatx4 v = {oacc[ob][4 * j] * inv * vs[c0], oacc[ob][4 * j + 1] * inv * vs[c0 + 1],
                             oacc[ob][4 * j + 2] * inv * vs[c0 + 2],
                             oacc[ob][4 * j + 3] * inv * vs[c0 + 3]};
                *reinterpret_cast<bf16x4*>(orow + c0) = __builtin_convertvector(v, bf16x4);
            }
        if (LSE != nullptr && hh == 0)
            LSE[(int64_t)bh * N + q_row] = (m - 8.f + log2f(l_tot)) * kLn2;
    }
}

// Token repair, the listed keys in every row: grid (ceil(N / 512), B*H), 4 waves, each
// taking 4 blocks of 32 rows in turn.  The listed keys are staged in LDS in groups of
// 128 (codes and exact rows; once per workgroup when there are at most 128), their V^T
// codes read from the quantiser's gathered copy (ld `ldr`).  For each key a wave forms
// both logits: t^ from the codes exactly as the main loop formed it, t~ from the exact
// row (Q codes widened to bf16 against it).  It keeps an integer maximum M', starting at
// ceil(log2 L) (no code logit exceeds log2 L) and raised only when an exact logit exceeds
// it (every rescale a power of two), and accumulates
// dA = sum (e4m3(2^(8+t~-M')) - e4m3(2^(8+t^-M'))) v8 on the fp8 matrix cores and
// dl = sum 2^(8+t~-M') - 2^(8+t^-M').  With u = 2^(M' - 8) / L, L = e^lse of the main
// kernel:  O' = (O + u vs dA) / (1 + u dl),   lse' = lse + ln(1 + u dl).
template <int D>
__global__ __launch_bounds__(256, 2) void fwd_fp8_keyfix_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const __bf16* __restrict__ K,
    const uint8_t* __restrict__ VSEL, const float* __restrict__ QS, const float* __restrict__ KS,
    const float* __restrict__ VS, const int32_t* __restrict__ KSEL,
    const int32_t* __restrict__ QSEL, int NREP, int ldr, int H, int N, float c2,
    __bf16* __restrict__ O, float* __restrict__ LSE) {
    constexpr int NWF = 4, QPW = 4, BC = 64, GT = 2, KB = BC / 32, NQC = D / 64, NOB = D / 32;
    constexpr int DC = D / 16;
    constexpr int KRPB = 256 / D;                       // code rows per 256-byte bank line
    constexpr int XU = D / 8;                           // 16-byte units per exact row
    constexpr int XRPL = 256 / (2 * D) > 0 ? 256 / (2 * D) : 1;
    __shared__ __attribute__((aligned(16))) uint8_t sk[GT][BC * D];
    __shared__ __attribute__((aligned(16))) __bf16 skx[GT][BC * D];
    __shared__ float ksl[GT * BC];
    __shared__ int ssel[GT * BC];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
    const int nblk = (N + JA_QK_BLOCK - 1) / JA_QK_BLOCK;
    const uint8_t* K8bh = K8 + (int64_t)bh * N * D;
    const __bf16* Kbh = K + (int64_t)bh * N * D;
    const uint8_t* Vsel = VSEL + (int64_t)bh * D * ldr;
    const int32_t* sel = KSEL + (int64_t)bh * NREP;
    auto kz = [&](int row) { return (row / KRPB) % DC; };
    auto xunit = [&](int row, int u) { return u ^ ((row / XRPL) % XU); };
    auto slot_of = [&](int kb, int a) { return kb * 32 + 16 * (a / 8) + 8 * hh + (a % 8); };

    // listed query rows of this workgroup's 512: recomputed with exact values already
    constexpr int WGR = NWF * QPW * 32;
    __shared__ uint32_t rmask[WGR / 32];
    if (tid < WGR / 32) rmask[tid] = 0;
    __syncthreads();
    for (int i = tid; i < NREP; i += 256) {
        const int r = QSEL[(int64_t)bh * NREP + i] - (int)blockIdx.x * WGR;
        if (r >= 0 && r < WGR) atomicOr(&rmask[r >> 5], 1u << (r & 31));
    }
    __syncthreads();

    const int ngroups = (NREP + GT * BC - 1) / (GT * BC);
    auto stage = [&](int g) {                           // listed keys g*128 .. -> LDS
        __syncthreads();                                // earlier readers
        if (tid < GT * BC) {
            const int r = g * GT * BC + tid;
            // (entries clamped below N; a negative one counts as an empty slot)
            const int key = r < NREP ? min(sel[r], N - 1) : -1;
            ssel[tid] = key;
            // empty slots: any finite positive factor, so that -inf logits stay -inf
            ksl[tid] = key >= 0 ? KS[(int64_t)bh * nblk + key / JA_QK_BLOCK] : 1.f;
        }
        __syncthreads();
        for (int x = tid; x < GT * BC * DC; x += 256) {
            const int kr = x / DC, u = x % DC, key = ssel[kr];
            const uint4 v = key >= 0 ? *reinterpret_cast<const uint4*>(K8bh + (int64_t)key * D + u * 16)
                                     : make_uint4(0, 0, 0, 0);
            const int tt = kr / BC, row = kr % BC;
            *reinterpret_cast<uint4*>(&sk[tt][row * D + (u ^ kz(row)) * 16]) = v;
        }
        for (int x = tid; x < GT * BC * XU; x += 256) {
            const int kr = x / XU, u = x % XU, key = ssel[kr];
            const uint4 v = key >= 0 ? *reinterpret_cast<const uint4*>(Kbh + (int64_t)key * D + u * 8)
                                     : make_uint4(0, 0, 0, 0);
            const int tt = kr / BC, row = kr % BC;
            *reinterpret_cast<uint4*>(&skx[tt][row * D + xunit(row, u) * 8]) = v;
        }
        __syncthreads();
    };
    if (ngroups == 1) stage(0);

#pragma unroll 1
    for (int qi = 0; qi < QPW; ++qi) {
        const int q_row = ((blockIdx.x * NWF + w) * QPW + qi) * 32 + r32;
        const int q_ld = min(q_row, N - 1);
        const float qsc2 = QS[(int64_t)bh * nblk + q_ld / JA_QK_BLOCK] * c2;
        intx8 qf[NQC];
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
            const uint4* p = reinterpret_cast<const uint4*>(Q8 + ((int64_t)bh * N + q_ld) * D +
                                                            64 * c + 32 * hh);
            const uint4 x0 = p[0], x1 = p[1];
            qf[c] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
        float* lp = LSE + (int64_t)bh * N + q_ld;
        const float lam = *lp * kLog2e;                 // log2 L >= every code logit t^
        __bf16* orow = O + (((int64_t)b * N + q_ld) * H + h) * D;

        floatx16 dacc[NOB];
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int a = 0; a < 16; ++a) dacc[ob][a] = 0.f;
        // M' starts at ceil(log2 L): no code term exceeds it, only exact logits can raise it
        float mr = ceilf(lam), dl = 0.f;
        for (int g = 0; g < ngroups; ++g) {
            if (ngroups > 1) stage(g);
            for (int tt = 0; tt < GT; ++tt) {
                const int r0 = (g * GT + tt) * BC;
                if (r0 >= NREP) break;
                // V^T codes of the gathered keys: row (channel) 32 i + r32, keys r0 + 16 u + 8 hh
                intx8 av[NOB];
#pragma unroll
                for (int i = 0; i < NOB; ++i) {
                    const uint8_t* vrow = Vsel + (int64_t)(32 * i + r32) * ldr + r0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint2 x = *reinterpret_cast<const uint2*>(vrow + 16 * u + 8 * hh);
                        av[i][2 * u] = (int)x.x;
                        av[i][2 * u + 1] = (int)x.y;
                    }
                }
                floatx16 sh[KB], sx[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int a = 0; a < 16; ++a) {
                        sh[kb][a] = 0.f;
                        sx[kb][a] = 0.f;
                    }
#pragma unroll
                for (int c = 0; c < NQC; ++c) {        // as the main loop: channels 64c + 32hh..
                    const int u0 = 4 * c + 2 * hh;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const int krow = kb * 32 + swap_bits23(r32);
                        const uint4 x0 = *reinterpret_cast<const uint4*>(
                            &sk[tt][krow * D + (u0 ^ kz(krow)) * 16]);
                        const uint4 x1 = *reinterpret_cast<const uint4*>(
                            &sk[tt][krow * D + ((u0 + 1) ^ kz(krow)) * 16]);
                        const intx8 ak = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                          (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                        sh[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ak, qf[c], sh[kb],
                                                                                0, 0, 0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int c16 = 0; c16 < D / 16; ++c16) {
                    const int c = c16 / 4, wq = 2 * (c16 % 4);
                    const bf16x8 bq = e4m3x8_to_bf16(qf[c][wq], qf[c][wq + 1]);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const int krow = kb * 32 + swap_bits23(r32);
                        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(
                            &skx[tt][krow * D + xunit(krow, rep_channel(c16, hh) / 8) * 8]);
                        sx[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, bq, sx[kb], 0, 0, 0);
                    }
                }
                const float* kslt = ksl + tt * BC;
                if (r0 + BC > NREP) {                   // the last, partial tile
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int a = 0; a < 16; ++a)
                            if (r0 + slot_of(kb, a) >= NREP) {
                                sh[kb][a] = -INFINITY;
                                sx[kb][a] = -INFINITY;
                            }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sx[kb][a]);
                mx *= qsc2;
                if (__ballot(mx > mr) != 0) {
                    const float m_new = fmaxf(mr, ceilf(wave_halves_max(mx)));
                    const float alpha = ldexpf(1.f, (int)(mr - m_new));
                    mr = m_new;
                    dl *= alpha;
#pragma unroll
                    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                        for (int a = 0; a < 16; ++a) dacc[ob][a] *= alpha;
                }
                const float bias = 8.f - mr;
                intx8 px, pn;
#pragma unroll
                for (int k = 0; k < 4 * KB; ++k) {
                    const int kb = k / 4, d = k % 4;
                    float p[4], q[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        p[e] = fast_exp2(fmaf(sx[kb][4 * d + e], qsc2, bias));
                        // the main loop's factor for this key, formed as the loop forms it
                        const float fk = qsc2 * kslt[slot_of(kb, 4 * d + e)];
                        q[e] = fast_exp2(fmaf(sh[kb][4 * d + e], fk, bias));
                    }
                    dl += ((p[0] + p[1]) + (p[2] + p[3])) - ((q[0] + q[1]) + (q[2] + q[3]));
                    const int wp = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                    px[k] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wp, true);
                    const int wn = __builtin_amdgcn_cvt_pk_fp8_f32(-q[0], -q[1], 0, false);
                    pn[k] = __builtin_amdgcn_cvt_pk_fp8_f32(-q[2], -q[3], wn, true);
                }
#pragma unroll
                for (int i = 0; i < NOB; ++i) {
                    dacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], px, dacc[i], 0,
                                                                             0, 0, 0, 0, 0);
                    dacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[i], pn, dacc[i], 0,
                                                                             0, 0, 0, 0, 0);
                }
            }
        }

        const float dlt = wave_halves_sum(dl);
        const int wr = q_row - (int)blockIdx.x * WGR;          // 0 <= wr < WGR
        if (q_row < N && !((rmask[wr >> 5] >> (wr & 31)) & 1u)) {
            const float u = exp2f(mr - 8.f - lam);
            const float den = 1.f + u * dlt;
            const float inv = 1.f / den;
            const float* vs = VS + (int64_t)bh * D;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c0 = ob * 32 + j * 8 + hh * 4;
                    const bf16x4 o4 = *reinterpret_cast<const bf16x4*>(orow + c0);
                    floatx4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = ((float)o4[e] + u * vs[c0 + e] * dacc[ob][4 * j + e]) * inv;
                    *reinterpret_cast<bf16x4*>(orow + c0) = __builtin_convertvector(v, bf16x4);
                }
            if (hh == 0) *lp = (lam + log2f(den)) * kLn2;
        }
    }
}

template <int D, bool HI>
hipError_t launch_d(const void* q8, const void* k8, const void* v8t, const float* qs,
                    const float* ks, const float* vs, const void* qh, const void* kh, int B,
                    int H, int N, int64_t ldv, float softmax_scale, void* o, float* lse,
                    hipStream_t stream) {
    constexpr int NW = D == 128 ? FP8_NW128 : 4;
    constexpr int BR = NW * 32;
    const int n_qtiles = (N + BR - 1) / BR;
    const int total = n_qtiles * B * H;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, HI>), dim3(total), dim3(NW * 64), 0, stream,
                       static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                       static_cast<const uint8_t*>(v8t), qs, ks, vs,
                       static_cast<const __bf16*>(qh), static_cast<const __bf16*>(kh), H, N, ldv,
                       softmax_scale * kLog2e, static_cast<__bf16*>(o), lse, n_qtiles, total);
    return hipGetLastError();
}

// split-KV: whole rounds of query tiles over all keys, the last round's `tail` tiles as
// n_split key ranges each, then the merge of the split tiles
template <int D, bool HI>
hipError_t launch_split_d(const void* q8, const void* k8, const void* v8t, const float* qs,
                          const float* ks, const float* vs, const void* qh, const void* kh, int B,
                          int H, int N, int64_t ldv, float softmax_scale, int n_split, int tail,
                          float* o_part, float* lse_part, void* o, float* lse,
                          hipStream_t stream) {
    constexpr int NW = D == 128 ? FP8_NW128 : 4;
    constexpr int BR = NW * 32;
    constexpr int RPB = 256 / (D / 4);
    const int n_qtiles = (N + BR - 1) / BR;
    const int n_full = n_qtiles * B * H - tail;
    const int total = n_full + tail * n_split;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, HI, false, true>), dim3(total), dim3(NW * 64), 0,
                       stream, static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                       static_cast<const uint8_t*>(v8t), qs, ks, vs,
                       static_cast<const __bf16*>(qh), static_cast<const __bf16*>(kh), H, N, ldv,
                       softmax_scale * kLog2e, static_cast<__bf16*>(o), lse, n_qtiles, total,
                       nullptr, nullptr, nullptr, nullptr, 0, n_split, o_part, lse_part, n_full);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((splitkv_merge_kernel<D, BR>), dim3(tail * (BR / RPB)), dim3(256), 0,
                       stream, o_part, lse_part, n_split, n_full, n_qtiles, H, N,
                       static_cast<__bf16*>(o), lse);
    return hipGetLastError();
}

template <int D>
hipError_t launch_repair_d(const void* q8, const void* k8, const void* v8t, const float* qs,
                           const float* ks, const float* vs, const void* q, const void* k,
                           const int32_t* q_sel, const int32_t* k_sel, const void* v8t_sel,
                           int n_repair, int B, int H, int N, int64_t ldv, float softmax_scale,
                           void* o, float* lse, hipStream_t stream) {
    if (n_repair == 0)
        return launch_d<D, false>(q8, k8, v8t, qs, ks, vs, nullptr, nullptr, B, H, N, ldv,
                                  softmax_scale, o, lse, stream);
    constexpr int NW = D == 128 ? FP8_NW128 : 4;
    constexpr int BR = NW * 32;
    const int n_qtiles = (N + BR - 1) / BR;
    const int total = n_qtiles * B * H;
    const int row_wgs = (n_repair + 31) / 32 * B * H;
    const float c2 = softmax_scale * kLog2e;
    // the main grid, then the listed rows' workgroups (dispatched last: they fill the
    // CUs the main grid's last round leaves idle); then the listed keys in every other row
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, false, true>), dim3(total + row_wgs), dim3(NW * 64),
                       0, stream, static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                       static_cast<const uint8_t*>(v8t), qs, ks, vs, nullptr, nullptr, H, N, ldv, c2,
                       static_cast<__bf16*>(o), lse, n_qtiles, total,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), q_sel, k_sel,
                       n_repair);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ldr = (n_repair + 63) / 64 * 64;
    hipLaunchKernelGGL(fwd_fp8_keyfix_kernel<D>, dim3((N + 511) / 512, B * H), dim3(256), 0,
                       stream, static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
                       static_cast<const __bf16*>(k), static_cast<const uint8_t*>(v8t_sel), qs,
                       ks, vs, k_sel, q_sel, n_repair, ldr, H, N, c2, static_cast<__bf16*>(o),
                       lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8_repair(const void* q8, const void* k8, const void* v8t,
                                 const float* q_scale, const float* k_scale, const float* v_scale,
                                 const void* q, const void* k, const int32_t* q_sel,
                                 const int32_t* k_sel, const void* v8t_sel, int n_repair, int B,
                                 int H, int N, int D, int64_t ldv, float softmax_scale, void* o,
                                 float* lse, hipStream_t stream) {
    return D == 64 ? launch_repair_d<64>(q8, k8, v8t, q_scale, k_scale, v_scale, q, k, q_sel,
                                         k_sel, v8t_sel, n_repair, B, H, N, ldv, softmax_scale, o,
                                         lse, stream)
                   : launch_repair_d<128>(q8, k8, v8t, q_scale, k_scale, v_scale, q, k, q_sel,
                                          k_sel, v8t_sel, n_repair, B, H, N, ldv, softmax_scale,
                                          o, lse, stream);
}

int fp8_splitkv_slots(int D, int mode) {
    // workgroups that run at once: the device's CUs times the occupancy the runtime gives
    // for the kernel actually launched
    int dev = 0, cus = 256, per = 1;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    constexpr int NW128 = FP8_NW128;
    hipError_t e;
    if (D == 64)
        e = mode == JA_FP8_SPLIT
                ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &per, fwd_fp8_kernel<64, 4, true, false, true>, 4 * 64, 0)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &per, fwd_fp8_kernel<64, 4, false, false, true>, 4 * 64, 0);
    else
        e = mode == JA_FP8_SPLIT
                ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &per, fwd_fp8_kernel<128, NW128, true, false, true>, NW128 * 64, 0)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                      &per, fwd_fp8_kernel<128, NW128, false, false, true>, NW128 * 64, 0);
    if (e != hipSuccess || per < 1) per = 1;
    return cus * per;
}

int fp8_splitkv_rows_per_tile(int D) { return D == 128 ? FP8_NW128 * 32 : 4 * 32; }

hipError_t launch_fwd_fp8_splitkv(const void* q8, const void* k8, const void* v8t,
                                  const float* q_scale, const float* k_scale,
                                  const float* v_scale, int B, int H, int N, int D, int64_t ldv,
                                  float softmax_scale, int mode, const void* q_hi,
                                  const void* k_hi, int n_split, int slots, float* o_part,
                                  float* lse_part, void* o, float* lse, hipStream_t stream) {
    const int tiles = (N + 63) / 64;                        // 64-key tiles
    n_split = n_split < tiles ? n_split : tiles;            // every key range non-empty
    const int br = fp8_splitkv_rows_per_tile(D);
    const int units = (N + br - 1) / br * B * H;
    const int tail = units % slots;                         // tiles of the last round
    if (n_split <= 1 || tail == 0)
        return launch_fwd_fp8(q8, k8, v8t, q_scale, k_scale, v_scale, B, H, N, D, ldv,
                              softmax_scale, mode, q_hi, k_hi, o, lse, stream);
    if (mode == JA_FP8_SPLIT)
        return D == 64 ? launch_split_d<64, true>(q8, k8, v8t, q_scale, k_scale, v_scale, q_hi,
                                                  k_hi, B, H, N, ldv, softmax_scale, n_split,
                                                  tail, o_part, lse_part, o, lse, stream)
                       : launch_split_d<128, true>(q8, k8, v8t, q_scale, k_scale, v_scale, q_hi,
                                                   k_hi, B, H, N, ldv, softmax_scale, n_split,
                                                   tail, o_part, lse_part, o, lse, stream);
    return D == 64 ? launch_split_d<64, false>(q8, k8, v8t, q_scale, k_scale, v_scale, nullptr,
                                               nullptr, B, H, N, ldv, softmax_scale, n_split,
                                               tail, o_part, lse_part, o, lse, stream)
                   : launch_split_d<128, false>(q8, k8, v8t, q_scale, k_scale, v_scale, nullptr,
                                                nullptr, B, H, N, ldv, softmax_scale, n_split,
                                                tail, o_part, lse_part, o, lse, stream);
}

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale,
                          const float* k_scale, const float* v_scale, int B, int H, int N, int D,
                          int64_t ldv, float softmax_scale, int mode, const void* q_hi,
                          const void* k_hi, void* o, float* lse, hipStream_t stream) {
    if (mode == JA_FP8_SPLIT)
        return D == 64 ? launch_d<64, true>(q8, k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi, B,
                                            H, N, ldv, softmax_scale, o, lse, stream)
                       : launch_d<128, true>(q8, k8, v8t, q_scale, k_scale, v_scale, q_hi, k_hi,
                                             B, H, N, ldv, softmax_scale, o, lse, stream);
    return D == 64 ? launch_d<64, false>(q8, k8, v8t, q_scale, k_scale, v_scale, nullptr, nullptr,
                                         B, H, N, ldv, softmax_scale, o, lse, stream)
                   : launch_d<128, false>(q8, k8, v8t, q_scale, k_scale, v_scale, nullptr, nullptr,
                                          B, H, N, ldv, softmax_scale, o, lse, stream);
}

}  // namespace ja

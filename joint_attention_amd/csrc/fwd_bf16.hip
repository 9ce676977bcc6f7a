// Joint attention forward, bf16 operands, fp32 accumulation, online softmax (gfx950).
//
// O = softmax(Q K^T * scale) V over the packed text + target + reference tokens
// (VisualGen FLUX 3 article, everytik.com translation, sections
// 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理 and 量化注意力与稀疏注意力).
//
// Work split.  One workgroup = 4 waves = 128 query rows of one (b, h); each wave owns
// 32 query rows for the whole key loop.  Keys are consumed in tiles of 64.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, wave64).  The wave computes the
// transposed scores S^T = K Q^T: operand A = 32 keys (from LDS), operand B = the
// wave's 32 queries (resident in VGPRs for the whole kernel).  In the 32x32 result
// each lane then holds ONE query column and 16 of its keys, so the softmax row max
// and row sum are mostly in-lane; only the two wave halves (which hold the same
// queries) are combined, with one v_permlane32_swap.  The PV product is computed as
// O^T = V^T P^T: A = V^T rows (channels, from LDS), B = P^T straight from the score
// registers converted to bf16 -- no LDS round trip for P.  For that, the key that
// feeds accumulator slot (a, half) must equal the key that B-operand slot (a, half)
// carries in the PV step; reading K rows in an order with bits 2 and 3 of the row
// index swapped makes each lane's 8 scores of a 16-key step 8 consecutive keys.
//
// LDS.  K tile [64 keys][D] and V^T tile [D][64 keys], 16-byte chunks XOR-swizzled by
// row so the 16-byte MFMA operand reads of 32 different rows are bank-conflict free.
// The next tile's global loads are issued into registers before the current tile's
// MFMAs and written to LDS after them.
#include "ja_device.h"
#include "ja_launch.h"

namespace ja {
namespace {

constexpr int BR = 128;          // query rows per workgroup
constexpr int BC = 64;           // keys per tile
constexpr int NTHREADS = 256;

__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(NTHREADS, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ VT,
    int H, int N, int64_t ldv, float c2, __bf16* __restrict__ O, float* __restrict__ LSE,
    int n_qtiles, int total) {
    constexpr int DC = D / 8;            // 16-byte chunks per K row
    constexpr int NQC = D / 16;          // k-steps of the QK product
    constexpr int NOB = D / 32;          // 32-channel blocks of the output
    constexpr int KCH = BC * DC / NTHREADS;
    constexpr int VCH = D * (BC / 8) / NTHREADS;
    __shared__ __attribute__((aligned(16))) __bf16 sk[BC * D];
    __shared__ __attribute__((aligned(16))) __bf16 sv[D * BC];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r32 = lane & 31, hh = lane >> 5;
    const int wg = xcd_remap(blockIdx.x, total);
    const int bh = wg / n_qtiles, qt = wg - bh * n_qtiles;
    const int b = bh / H, h = bh - b * H;
    const __bf16* Qbh = Q + (int64_t)bh * N * D;
    const __bf16* Kbh = K + (int64_t)bh * N * D;
    const __bf16* Vbh = VT + (int64_t)bh * D * ldv;

    const int q_row = qt * BR + w * 32 + r32;
    const int q_ld = min(q_row, N - 1);
    bf16x8 qf[NQC];
#pragma unroll
    for (int c = 0; c < NQC; ++c)
        qf[c] = *reinterpret_cast<const bf16x8*>(Qbh + (int64_t)q_ld * D + 16 * c + 8 * hh);

    floatx16 oacc[NOB];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
        for (int a = 0; a < 16; ++a) oacc[ob][a] = 0.f;
    // m: the row maximum used as the exponent offset (base-2 units).  It is raised only
    // when a tile's maximum exceeds it by more than kLazy, so most tiles skip the
    // rescale of O; the numerators 2^(t - m) then stay below 2^kLazy.
    constexpr float kLazy = 8.f;
    float m = -INFINITY, l = 0.f;

    const int nkt = (N + BC - 1) / BC;
    const int nfull = N / BC;             // tiles with all 64 keys inside the sequence
    uint4 kreg[KCH], vreg[VCH];

    auto load_full = [&](int kt) {
        const int k0 = kt * BC;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / DC, ch = idx % DC;
            kreg[i] = *reinterpret_cast<const uint4*>(Kbh + (int64_t)(k0 + row) * D + ch * 8);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / (BC / 8), ch = idx % (BC / 8);
            vreg[i] = *reinterpret_cast<const uint4*>(Vbh + (int64_t)row * ldv + k0 + ch * 8);
        }
    };
    // last, partial tile: keys >= N read as zero (K rows and V^T columns)
    auto load_tail = [&](int kt) {
        const int k0 = kt * BC;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / DC, ch = idx % DC;
            const int key = k0 + row;
            kreg[i] = make_uint4(0, 0, 0, 0);
            if (key < N)
                kreg[i] = *reinterpret_cast<const uint4*>(Kbh + (int64_t)key * D + ch * 8);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / (BC / 8), ch = idx % (BC / 8);
            const int key = k0 + ch * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (key < N) {
                // key < N and key % 8 == 0 keep key + 8 <= ldv (ldv % 16 == 0)
                v = *reinterpret_cast<const uint4*>(Vbh + (int64_t)row * ldv + key);
                uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (key + 2 * e >= N) wv[e] = 0;
                    else if (key + 2 * e + 1 >= N) wv[e] &= 0xFFFFu;
                }
                v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            vreg[i] = v;
        }
    };
    auto load_tile = [&](int kt) {
        if (kt < nfull) load_full(kt);
        else load_tail(kt);
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / DC, ch = idx % DC;
            *reinterpret_cast<uint4*>(&sk[row * D + ((ch ^ (row % DC)) * 8)]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int idx = tid + i * NTHREADS, row = idx / (BC / 8), ch = idx % (BC / 8);
            *reinterpret_cast<uint4*>(&sv[row * BC + ((ch ^ ((row >> 1) & 7)) * 8)]) = vreg[i];
        }
    };

    auto tile = [&](int kt) {
        // S^T for two 32-key blocks
        floatx16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int krow = kb * 32 + swap_bits23(r32);
#pragma unroll
            for (int c = 0; c < NQC; ++c) {
                const int u = 2 * c + hh;
                const bf16x8 av =
                    *reinterpret_cast<const bf16x8*>(&sk[krow * D + ((u ^ (krow % DC)) * 8)]);
                if (c == 0) {
                    const floatx16 zero = {};
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[c], zero, 0, 0, 0);
                } else {
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[c], s[kb], 0, 0, 0);
                }
            }
        }
        if (kt >= nfull) {                        // last, partial tile (uniform branch)
            const int k0 = kt * BC;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int key = k0 + kb * 32 + 16 * (a / 8) + 8 * hh + (a % 8);
                    if (key >= N) s[kb][a] = -INFINITY;
                }
        }

        // online softmax in base 2: t = s * c2 with c2 = scale * log2(e)
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s[kb][a]);
        mx = wave_halves_max(mx) * c2;
        if (__ballot(mx > m + kLazy) != 0) {       // wave-uniform: some row's max grew a lot
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int a = 0; a < 16; ++a) oacc[ob][a] *= alpha;
        }

        bf16x8 pf[4];
        const float nm = -m;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    floatx2 pr = {fast_exp2(fmaf(s[kb][8 * u + 2 * e], c2, nm)),
                                  fast_exp2(fmaf(s[kb][8 * u + 2 * e + 1], c2, nm))};
                    const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
                    // row sum of the bf16 numerators that feed the P.V product
                    l = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.f, (__bf16)1.f}, l,
                                                        false);
                    pf[2 * kb + u][2 * e] = pb[0];
                    pf[2 * kb + u][2 * e + 1] = pb[1];
                }

        // O^T += V^T P^T
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) {
            const int vrow = ob * 32 + r32;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int u = 2 * t + hh;
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(
                    &sv[vrow * BC + ((u ^ ((vrow >> 1) & 7)) * 8)]);
                oacc[ob] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[t], oacc[ob], 0, 0, 0);
            }
        }
    };

    load_tile(0);
    for (int kt = 0; kt < nkt; ++kt) {
        store_tile();
        __syncthreads();
        if (kt + 1 < nkt) load_tile(kt + 1);
        tile(kt);
        __syncthreads();
    }

    const float l_tot = wave_halves_sum(l);
    const float inv = 1.f / l_tot;
    if (q_row < N) {
        __bf16* orow = O + (((int64_t)b * N + q_row) * H + h) * D;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                floatx4 v = {oacc[ob][4 * j] * inv, oacc[ob][4 * j + 1] * inv,
                             oacc[ob][4 * j + 2] * inv, oacc[ob][4 * j + 3] * inv};
                *reinterpret_cast<bf16x4*>(orow + ob * 32 + j * 8 + hh * 4) =
                    __builtin_convertvector(v, bf16x4);
            }
        if (LSE != nullptr && hh == 0)
            LSE[(int64_t)bh * N + q_row] = (m + log2f(l_tot)) * kLn2;
    }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* vt, int B, int H, int N,
                    int64_t ldv, float softmax_scale, void* o, float* lse, hipStream_t stream) {
    const int n_qtiles = (N + BR - 1) / BR;
    const int total = n_qtiles * B * H;
    hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(total), dim3(NTHREADS), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(vt), H, N, ldv, softmax_scale * kLog2e,
                       static_cast<__bf16*>(o), lse, n_qtiles, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* vt, int B, int H, int N,
                           int D, int64_t ldv, float softmax_scale, void* o, float* lse,
                           hipStream_t stream) {
    return D == 64 ? launch_d<64>(q, k, vt, B, H, N, ldv, softmax_scale, o, lse, stream)
                   : launch_d<128>(q, k, vt, B, H, N, ldv, softmax_scale, o, lse, stream);
}

}  // namespace ja

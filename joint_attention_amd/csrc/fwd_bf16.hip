// Joint attention forward, bf16 operands, fp32 accumulation, online softmax (gfx950).
//
// O = softmax(Q K^T * scale) V over the packed text + target + reference tokens
// (VisualGen FLUX 3 article, everytik.com translation, sections
// 使用 TensorRT LLM VisualGen 进行 FLUX 3 推理 and 量化注意力与稀疏注意力).
//
// Work split.  One workgroup = 8 waves = 256 query rows of one (b, h) (head size 64: 4
// waves, 128 rows); each wave owns one 32-row query block for the whole key loop, two
// waves share a SIMD, and Q, O, two score tiles and two P tiles stay in its 256 VGPRs.
// Keys are consumed in tiles of BC = 32, loaded once per workgroup into LDS.
//
// Variants of the same kernel: GATHER reads Q and K (and, in mode 1, V) in place from the
// per-stream tensors (no pack step for them); SPARSE visits only the key blocks that an input block mask
// allows; PARTIAL splits the keys of the last round's query tiles into ranges whose
// partial results splitkv_merge_kernel combines (split-KV).
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
// Software pipeline.  Iteration j runs the softmax of tile j on the vector ALU while
// the matrix cores run P(j-1) V(j-1) and Q K(j+1)^T; the three are independent, and
// the loop body is written as an explicit sequence of steps (one LDS operand read, one
// or two MFMAs and a slice of the softmax each) separated by scheduling fences.  K and
// V^T tiles are double-buffered in LDS with one barrier per iteration.  The packed
// variants load them straight from HBM into LDS (global_load_lds_dwordx4, issued after
// the barrier that frees the slot); the stream gather stages K and a token-major V
// tile in registers one iteration ahead, writes K linearly and transposes V through LDS.
// Chunks are XOR-swizzled by row so that every LDS access is conflict-free on gfx950
// (a read serves 256 bytes per clock: 16 lanes of a 16-byte read; a write 128 bytes: 8
// lanes of a 16-byte write); for the loaded tiles the swizzle is applied on the global
// side, so each chunk lands lane-linear.
//
// Softmax details.  Scores are scaled to base 2 (c2 = scale * log2 e) in the FMA that
// subtracts the running offset m.  m is raised (to the exact row maximum, combining the
// two lane halves) only when some lane's own maximum exceeds it by more than 16, so the
// cross-lane step and the rescale of O are rare; the numerators stay below 2^16.  The row
// sum accumulates the bf16-rounded numerators with v_dot2 (the same values that
// enter P V).
#include <mutex>
#include <type_traits>

#include "ja_device.h"
#include "ja_launch.h"
#include "splitkv_merge.h"

namespace ja {
namespace {

#ifndef FWD_NW
#define FWD_NW 8
#endif
// block-sparse D = 128: 128-row workgroups (two per CU), so that a workgroup visits exactly
// its own mask row's key blocks instead of the union of two rows'
#ifndef FWD_NW_SPARSE
#define FWD_NW_SPARSE 4
#endif
#ifndef FWD_QB
#define FWD_QB 1
#endif
#ifndef FWD_BC
#define FWD_BC 32
#endif
#ifndef FWD_LEAD
#define FWD_LEAD 2          // operand read distance, tiles loaded by DMA
#endif
#ifndef FWD_LEAD_GATHER
#define FWD_LEAD_GATHER 3   // the same for the register-staged stream gather
#endif
#ifndef FWD_TW
#define FWD_TW 3
#endif

__device__ inline int swap_bits23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// NW: waves per workgroup (each owns QB 32-row query blocks); BC: keys per tile.  With
// NW * QB = 8 one workgroup covers 256 query rows (every K/V tile loaded into LDS serves
// 256 rows) and fills a CU at two waves per SIMD; with NW * QB = 4 two 128-row workgroups
// share a CU (D = 64, and the block-sparse forward, whose workgroups then match its mask
// blocks).
// GATHER = 1: Q, K and V are read in place from the per-stream tensors of `st`
// (token-major [B][L_s][H][D]) instead of the packed Q, K (BHND) and V^T (BHDN); V tiles
// are then kept token-major in LDS and read with transposing LDS loads.
// GATHER = 2: Q and K are read in place from the streams (K tiles by LDS DMA, each key
// row being D contiguous elements of its stream's row), V^T from a packed copy (BHDN).
// SPARSE: only the key blocks that a block mask (uint8 [B][H][nqb][nkb], 128 x 128 blocks)
// allows for at least one of the workgroup's query blocks are visited; a wave whose own
// query block does not see a visited block gives it zero weight.  With a dispatch plan
// (ORDER, from sparse_plan_*_kernel below) workgroup position p runs query block ORDER[p]
// instead of p: the same work per workgroup, started in another order.
// PARTIAL (split-KV): the first n_full query tiles (whole rounds of workgroups over the
// CUs) run over all keys and write O as usual; for each later query tile the keys are cut
// into n_split ranges of whole tiles, one workgroup per (query tile, range), each writing
// its normalised fp32 partial output and lse (OP [part][BR][D], LP [part][BR], part =
// (tile - n_full) * n_split + range) for the merge kernel below.
template <int D, int NW, int QB, int BC, int GATHER, bool SPARSE, bool PARTIAL = false>
__global__ __launch_bounds__(NW * 64, 8 / (NW * QB)) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ VT,
    const StreamTable st, const uint8_t* __restrict__ MASK, int H, int N, int64_t ldv, float c2,
    __bf16* __restrict__ O, float* __restrict__ LSE, int n_qtiles, int total,
    int n_split = 1, float* __restrict__ OP = nullptr, float* __restrict__ LP = nullptr,
    int n_full = 0, const int32_t* __restrict__ ORDER = nullptr) {
    static_assert(GATHER >= 0 && GATHER <= 2, "gather mode");
    static_assert(!(SPARSE && (GATHER || PARTIAL)), "the block-sparse forward runs alone");
    constexpr bool GQK = GATHER != 0;            // Q and K read from the streams
    constexpr bool GV = GATHER == 1;             // V read from the streams (transposed in LDS)
    constexpr int NTHREADS = NW * 64;
    constexpr int BR = NW * QB * 32;             // query rows per workgroup
    constexpr int KB = BC / 32;                  // 32-key blocks per tile
    constexpr int DC = D / 8;                    // 16-byte chunks per K row
    constexpr int NQC = D / 16;                  // k-steps of the QK product
    constexpr int NOB = D / 32;                  // 32-channel blocks of the output
    constexpr int VCPR = BC / 8;                 // 16-byte chunks per V^T row
    constexpr int VRPB = 256 / (2 * BC);         // V^T rows per 256 bytes (all 64 banks)
    static_assert(VCPR >= 4, "the V^T swizzle below uses two chunk bits");
    constexpr int TILE_ELEMS = BC * D;           // bf16 elements of one K or V^T tile
    constexpr int LOADS = TILE_ELEMS * 2 / 1024 / (NTHREADS / 64);   // 1 KB loads per wave
    static_assert(LOADS >= 1, "tile smaller than one load per wave");
    constexpr float kLazy = 16.f;
    constexpr int GSEG = D / 32;                 // 64-byte segments per token-major V row
    constexpr int GRPL = 128 / D;                // token-major V rows per 256-byte line
    __shared__ __attribute__((aligned(1024))) __bf16 sk0[TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sk1[TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sv0[TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 sv1[TILE_ELEMS];
    // GATHER = 1: token-major V tiles, transposed into sv0 / sv1 one iteration later
    __shared__ __attribute__((aligned(1024))) __bf16 st0[GV ? TILE_ELEMS : 8];
    __shared__ __attribute__((aligned(1024))) __bf16 st1[GV ? TILE_ELEMS : 8];

    // V^T rows: 16-byte chunk u of row r sits at chunk u ^ vswz(r).  A 16-byte operand
    // read serves 16 rows at once (VRPB rows per 256-byte bank line: (r / VRPB) picks
    // distinct chunks), a 16-byte LDS write 8 rows in a 128-byte window (the (r / 2) bit
    // separates rows r and r + 2, which share that window's banks)
    auto vswz = [](int r) { return ((r / VRPB) % VCPR) ^ (((r / 2) & 1) << 1); };
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept scalar
    const int r32 = lane & 31, hh = lane >> 5;
    // PARTIAL: the whole-round workgroups and the split ones are renumbered separately, so
    // that both spread evenly over the XCDs (n_full is a multiple of the slot count)
    const int bid = blockIdx.x;
    const int wg = !PARTIAL ? xcd_remap(bid, total)
                   : bid < n_full ? xcd_remap(bid, n_full)
                                  : n_full + xcd_remap(bid - n_full, total - n_full);
    // consecutive workgroups share (b, h); in PARTIAL those past n_full are the ranges of
    // one query tile
    int unit = wg, split = 0;
    // SPARSE with a dispatch plan: position wg runs query block ORDER[wg] (clamped, so that
    // a plan that is not a permutation can only leave rows unwritten, never reach outside)
    if (SPARSE && ORDER != nullptr) unit = min(max(ORDER[wg], 0), total - 1);
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
    const __bf16* Qbh = Q + (int64_t)bh * N * D;
    const __bf16* Kbh = K + (int64_t)bh * N * D;
    const __bf16* Vbh = VT + (int64_t)bh * D * ldv;
    int nkt = (N + BC - 1) / BC;
    int t_begin = 0;                             // PARTIAL: first key tile of this range
    if (PARTIAL && part_wg) {
        // n_split <= the number of key tiles (the launcher clamps it): no range is empty
        const int all = nkt;
        t_begin = (int)((int64_t)split * all / n_split);
        nkt = (int)((int64_t)(split + 1) * all / n_split) - t_begin;
    }

    // ---- SPARSE: table of the active 128-key blocks (block index | flags << 16, one flag
    //      per query block of the workgroup), compacted by wave 0 with ballots
    constexpr int TPB = JA_SPARSE_BLOCK / BC;    // key tiles per mask block
    __shared__ int ktab[SPARSE ? JA_SPARSE_MAX_N / JA_SPARSE_BLOCK : 1];
    __shared__ int ktab_n, ktab_rot;
    int sp_group = 0;                            // this wave's query block in the workgroup
    // SPARSE: the visit starts at the first active block at or past 2 x (first query block)
    // and wraps around.  Workgroups that run together on an XCD hold neighbouring query
    // blocks, so they move through the key blocks together and share them in L2 (in the
    // given order every one starts at block 0 and they drift apart).  A workgroup that
    // sees every block keeps the plain order; a last block that runs past N stays last
    // (only the full blocks n_rot rotate), so that only the last tiles need the tail mask.
    int rot = 0, n_rot = 0;
    if constexpr (SPARSE) {
        constexpr int QBW = BR / JA_SPARSE_BLOCK;
        static_assert(QBW >= 1 && QBW * JA_SPARSE_BLOCK == BR, "workgroup rows per mask block");
        const int nb = (N + JA_SPARSE_BLOCK - 1) / JA_SPARSE_BLOCK;
        const int qb0 = qt * QBW;
        const int start = (2 * qb0) % nb;
        sp_group = (w * QB * 32) / JA_SPARSE_BLOCK;
        if (w == 0) {
            int count = 0, below_start = 0;
            for (int base = 0; base < nb; base += 64) {
                const int kb = base + lane;
                int flags = 0;
                if (kb < nb) {
#pragma unroll
                    for (int g = 0; g < QBW; ++g)
                        if (qb0 + g < nb && MASK[((int64_t)bh * nb + qb0 + g) * nb + kb] != 0)
                            flags |= 1 << g;
                }
                const uint64_t bal = __ballot(flags != 0);
                below_start += __popcll(__ballot(flags != 0 && kb < start));
                if (flags) {
                    const int below = __builtin_amdgcn_mbcnt_hi(
                        (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                    ktab[count + below] = kb | (flags << 16);
                }
                count += __popcll(bal);
            }
            if (lane == 0) {
                ktab_n = count;
                ktab_rot = below_start;
            }
        }
        __syncthreads();
        const int nact = ktab_n;
        const bool tail_last = nact > 0 && (N % JA_SPARSE_BLOCK) != 0 &&
                               (ktab[nact - 1] & 0xFFFF) == nb - 1;
        n_rot = nact - (tail_last ? 1 : 0);
        rot = (nact < nb && ktab_rot < n_rot) ? ktab_rot : 0;
        nkt = nact * TPB;
        if (nact > 0) {
            // only the last mask block runs past N: drop its tiles that start at or past N
            const int last = (ktab[nact - 1] & 0xFFFF) * JA_SPARSE_BLOCK;
            nkt -= TPB - min(TPB, (N - last + BC - 1) / BC);
        }
        if (nkt == 0) {
            // no row of this workgroup sees any key: O = 0, lse = -inf
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int q_row = qt * BR + w * (QB * 32) + r32 + 32 * qb;
                if (q_row < N) {
                    __bf16* orow = O + (((int64_t)b * N + q_row) * H + h) * D;
#pragma unroll
                    for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            *reinterpret_cast<uint2*>(orow + ob * 32 + j * 8 + hh * 4) =
                                make_uint2(0, 0);
                    if (LSE != nullptr && hh == 0) LSE[(int64_t)bh * N + q_row] = -INFINITY;
                }
            }
            return;
        }
    }
    // keys of this workgroup end at kend (N, or the end of a split range).  A workgroup with
    // one key tile runs two, the second masked out entirely (its P is exactly zero), so that
    // every workgroup takes the one pipelined path (a separate one-tile path kept values
    // live across both and cost registers).  (SPARSE: one visited tile is only possible in
    // the last mask block, and its next tile starts at or past N.)
    const int kend = (PARTIAL && part_wg) ? min(N, (t_begin + nkt) * BC) : N;
    nkt = max(nkt, 2);
    auto tile_k0 = [&](int t) -> int {           // first key of (visited) key tile t
        if constexpr (SPARSE) {
            int e = t / TPB;
            if (e < n_rot) {
                e += rot;
                if (e >= n_rot) e -= n_rot;
            }
            return (ktab[e] & 0xFFFF) * JA_SPARSE_BLOCK + (t % TPB) * BC;
        }
        return (t_begin + t) * BC;
    };
    auto tile_on = [&](int t) -> bool {          // SPARSE: this wave's query block sees tile t
        if constexpr (SPARSE) {
            int e = t / TPB;
            if (e < n_rot) {
                e += rot;
                if (e >= n_rot) e -= n_rot;
            }
            return ((ktab[e] >> (16 + sp_group)) & 1) != 0;
        }
        return true;
    };

    // GATHER: packed token n -> its row (b, n - off[s], h) of stream s's tensor
    auto stream_of = [&](int n) {
        int s = 0;
        for (int i = 1; i < st.n; ++i)
            if (n >= st.off[i]) s = i;           // zero-length streams share the next start
        return s;
    };
    auto stream_row = [&](const void* const* src, int s, int n) -> const __bf16* {
        const int64_t L = st.off[s + 1] - st.off[s];
        return static_cast<const __bf16*>(src[s]) +
               (((int64_t)b * L + (n - st.off[s])) * H + h) * (int64_t)D;
    };
    const int64_t row_pitch = GQK ? (int64_t)H * D : D;   // elements between Q / K tokens
    // GATHER: tiles are visited in order, so each tensor keeps a cursor on the stream that
    // holds its current tile; the stream table is read only when a tile crosses into the
    // next stream (reads of it inside the loop would also stall the LDS-operand waits)
    struct Cursor {
        int s, start, end;               // stream s holds packed tokens [start, end)
        const __bf16* row0;              // its row for packed token `start`
        int next;                        // packed token whose row `ptr` is (-1: none)
        const __bf16* ptr;
    };
    auto cursor_init = [&](const void* const* src) {
        Cursor c{0, 0, (int)st.off[1], nullptr, 0, nullptr};
        if (GQK) c.row0 = c.ptr = stream_row(src, 0, 0);
        return c;
    };
    auto advance = [&](Cursor& c, const void* const* src, int key) {   // key >= c.start
        while (key >= c.end && c.s + 1 < st.n) {
            ++c.s;
            c.start = c.end;
            c.end = (int)st.off[c.s + 1];
            c.row0 = stream_row(src, c.s, c.start);
            c.next = -1;
        }
    };
    // the row of packed token k0 (a tile's first key) when the whole tile lies in one
    // stream, else nullptr (it straddles streams or N); tiles come in order, so the row
    // pointer normally just moves on by one tile (a multiply only after a jump)
    auto tile_base = [&](Cursor& c, const void* const* src, int k0) -> const __bf16* {
        advance(c, src, k0);                                    // wave-uniform
        if (k0 + BC > c.end) return nullptr;
        if (k0 != c.next) c.ptr = c.row0 + (int64_t)(k0 - c.start) * row_pitch;
        const __bf16* p = c.ptr;
        c.ptr = p + BC * row_pitch;
        c.next = k0 + BC;
        return p;
    };
    Cursor kcur = cursor_init(st.k), vcur = cursor_init(st.v);

    // ---- K / V^T tile placement: lane `lane` of wave w owns tile bytes
    //      (w*LOADS + i) * 1024 + 16 * lane; the swizzle is inverted on the global side,
    //      so each 16-byte chunk lands lane-linear (by DMA, or by one linear LDS store on
    //      the register-staged path)
    auto k_row = [&](int i) { return ((w * LOADS + i) * 1024 + lane * 16) / (2 * D); };
    auto k_chunk = [&](int i) {
        const int off = (w * LOADS + i) * 1024 + lane * 16;
        return ((off % (2 * D)) / 16) ^ ((off / (2 * D)) % DC);
    };
    auto v_row = [&](int i) {
        const int off = (w * LOADS + i) * 1024 + lane * 16;
        return GV ? off / (2 * D) : off / (2 * BC);
    };
    auto v_chunk = [&](int i) {
        const int off = (w * LOADS + i) * 1024 + lane * 16;
        if constexpr (GV) {
            // token-major V tile: the 64-byte segments of each key row are rotated by
            // (key / GRPL) % GSEG (conflict-free for the transposing reads)
            return ((off % (2 * D)) / 16) ^ ((((off / (2 * D)) / GRPL) % GSEG) * 4);
        }
        return ((off % (2 * BC)) / 16) ^ vswz(off / (2 * BC));
    };
    uint32_t k_off[LOADS], v_off[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        k_off[i] = (uint32_t)(k_row(i) * row_pitch + k_chunk(i) * 8) * 2u;
        v_off[i] = GV ? (uint32_t)(v_row(i) * row_pitch + v_chunk(i) * 8) * 2u
                          : (uint32_t)(v_row(i) * (int)ldv + v_chunk(i) * 8) * 2u;
    }
    uint4 kst[LOADS], vst[LOADS];                 // staged tiles (global -> registers)
    auto load_k = [&](int kt) {                  // GATHER = 1 only (the others load K by DMA)
        const int k0 = tile_k0(kt);
        if constexpr (GV) {
            if (const __bf16* row = tile_base(kcur, st.k, k0)) {  // the tile lies in one stream
                const char* base = reinterpret_cast<const char*>(row);
#pragma unroll
                for (int i = 0; i < LOADS; ++i)
                    kst[i] = *reinterpret_cast<const uint4*>(base + k_off[i]);
            } else {                                            // straddles streams or N
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    const int key = min(k0 + k_row(i), N - 1);  // rows past N: any finite row
                    kst[i] = *reinterpret_cast<const uint4*>(
                        stream_row(st.k, stream_of(key), key) + k_chunk(i) * 8);
                }
            }
        }
    };
    auto load_v = [&](int kt) {
        const int k0 = tile_k0(kt);
        if constexpr (GV) {
            // token-major rows as for K; rows past N repeat row N-1 (finite, and their
            // probabilities are exactly zero)
            if (const __bf16* row = tile_base(vcur, st.v, k0)) {
                const char* base = reinterpret_cast<const char*>(row);
#pragma unroll
                for (int i = 0; i < LOADS; ++i)
                    vst[i] = *reinterpret_cast<const uint4*>(base + v_off[i]);
            } else {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    const int key = min(k0 + v_row(i), N - 1);
                    vst[i] = *reinterpret_cast<const uint4*>(
                        stream_row(st.v, stream_of(key), key) + v_chunk(i) * 8);
                }
            }
            return;
        }
        if (k0 + BC <= N) {
            const char* base = reinterpret_cast<const char*>(Vbh + k0);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                vst[i] = *reinterpret_cast<const uint4*>(base + v_off[i]);
        } else {
            // last tile: columns >= N read as zero (the row may be padded with anything)
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int c0 = k0 + v_chunk(i) * 8;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c0 < N) {
                    // c0 < N, c0 % 8 == 0 and ldv % 16 == 0 keep c0 + 8 <= ldv
                    v = *reinterpret_cast<const uint4*>(Vbh + (int64_t)v_row(i) * ldv + c0);
                    uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (c0 + 2 * e >= N) wv[e] = 0;
                        else if (c0 + 2 * e + 1 >= N) wv[e] &= 0xFFFFu;
                    }
                    v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                }
                vst[i] = v;
            }
        }
    };
    auto store_k = [&](__bf16* slot) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            *reinterpret_cast<uint4*>(slot + (w * LOADS + i) * 512 + lane * 8) = kst[i];
    };
    // GATHER = 1: V^T chunk (row c, keys 8u .. 8u + 7) of a token-major tile in `ts`, one per
    // thread: in each 16-lane group, lane k points at key 8u + 4 half + (k >> 2), channels
    // 4 (k & 3) .. + 3 of the group's 16 channels; the transposing read hands lane r the 4
    // keys of channel c0 + r.  Written later to `vs` in the V^T layout of the operand reads
    // (the write waits for the reads, so it is placed a few MFMA steps after them).
    static_assert(!GV || NTHREADS * 8 == TILE_ELEMS,
                  "the transpose moves one 16-byte V^T chunk per thread");
    auto transpose_read = [&](const __bf16* ts) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        const int grp = tid >> 4, i16 = tid & 15;
        const int c0 = (grp % (D / 16)) * 16, u = grp / (D / 16);
        const int a = i16 & 3, jj = i16 >> 2;
        v4s r[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int key = 8 * u + 4 * half + jj;               // (key / GRPL) % GSEG
            const int byte = key * (2 * D) + (((c0 + 4 * a) * 2) ^ (((jj / GRPL) % GSEG) * 64));
            r[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(reinterpret_cast<const char*>(ts) +
                                                         byte));
        }
        return uint4{__builtin_bit_cast(uint2, r[0]).x, __builtin_bit_cast(uint2, r[0]).y,
                     __builtin_bit_cast(uint2, r[1]).x, __builtin_bit_cast(uint2, r[1]).y};
    };
    auto transpose_write = [&](const uint4& x, __bf16* vs) {
        const int grp = tid >> 4, i16 = tid & 15;
        const int row = (grp % (D / 16)) * 16 + i16, u = grp / (D / 16);
        *reinterpret_cast<uint4*>(vs + row * BC + ((u ^ vswz(row)) * 8)) = x;
    };
    auto store_v = [&](__bf16* slot) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            *reinterpret_cast<uint4*>(slot + (w * LOADS + i) * 512 + lane * 8) = vst[i];
    };

    // direct global -> LDS loads (gfx950 global_load_lds_dwordx4; not for GATHER = 1, whose
    // V goes through a transpose): each wave's 16-byte chunks land lane-linear in the slot,
    // the layout store_k / store_v write (the swizzle lives in the global offsets), with
    // no staging registers and no LDS store instructions
    constexpr bool DMA = !GV;
    auto dma16 = [&](const void* src, __bf16* dst) {
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    };
    auto dma_k = [&](int kt, __bf16* slot) {
        const int k0 = tile_k0(kt);
        if constexpr (GQK) {
            // stream rows: a tile inside one stream from the cursor's scalar base, one that
            // straddles streams (or N) row by row
            if (const __bf16* row = tile_base(kcur, st.k, k0)) {
                const char* base = reinterpret_cast<const char*>(row);
#pragma unroll
                for (int i = 0; i < LOADS; ++i) dma16(base + k_off[i], slot + (w * LOADS + i) * 512);
            } else {
#pragma unroll
                for (int i = 0; i < LOADS; ++i) {
                    const int key = min(k0 + k_row(i), N - 1);  // rows past N: any finite row
                    dma16(stream_row(st.k, stream_of(key), key) + k_chunk(i) * 8,
                          slot + (w * LOADS + i) * 512);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const char* src;
            if (k0 + BC <= N) {
                src = reinterpret_cast<const char*>(Kbh + (int64_t)k0 * D) + k_off[i];
            } else {
                const int key = min(k0 + k_row(i), N - 1);     // rows past N: any finite row
                src = reinterpret_cast<const char*>(Kbh + (int64_t)key * D + k_chunk(i) * 8);
            }
            dma16(src, slot + (w * LOADS + i) * 512);
        }
    };
    auto dma_v = [&](int kt, __bf16* slot) {
        const int k0 = tile_k0(kt);
        if (k0 + BC <= N) {
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                dma16(reinterpret_cast<const char*>(Vbh + k0) + v_off[i],
                      slot + (w * LOADS + i) * 512);
        } else {                                       // last tile: columns >= N zeroed
            load_v(kt);
            store_v(slot);
        }
    };
    // the DMA writes land in LDS asynchronously (counted by vmcnt): every wave waits for
    // its own before the barrier that hands the slot to the others
    auto dma_wait = [&]() {
        if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // ---- resident state
    const int q_base = qt * BR + w * (QB * 32) + r32;     // query row of block 0
    bf16x8 qf[QB][NQC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int q_ld = min(q_base + 32 * qb, N - 1);
        const __bf16* qrow = GQK ? stream_row(st.q, stream_of(q_ld), q_ld)
                                    : Qbh + (int64_t)q_ld * D;
#pragma unroll
        for (int c = 0; c < NQC; ++c)
            qf[qb][c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * hh);
    }
    floatx16 oacc[QB][NOB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int a = 0; a < 16; ++a) oacc[qb][ob][a] = 0.f;
    // m: row maximum used as the exponent offset (base 2), raised only when a tile's
    // maximum exceeds it by more than kLazy; l: running row sum (per lane half)
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
    }

    // ---- MFMA steps: one LDS operand read shared by QB MFMAs
    // PV step i = (t, ob): A = V^T rows ob*32.., keys 16t.. of the tile; B = P^T block t.
    // QK step i = (c, kb): A = K rows kb*32.. (bits 2/3 swapped), channels 16c..; B = Q.
    constexpr int NPV = 2 * KB * NOB;
    constexpr int NQK = NQC * KB;
    auto pv_operand = [&](const __bf16* vs, int i) {
        const int t = i / NOB, ob = i % NOB;
        const int vrow = ob * 32 + r32;
        const int u = 2 * t + hh;
        return *reinterpret_cast<const bf16x8*>(
            &vs[vrow * BC + ((u ^ vswz(vrow)) * 8)]);
    };
    auto qk_operand = [&](const __bf16* ks, int i) {
        const int c = i / KB, kb = i % KB;
        const int krow = kb * 32 + swap_bits23(r32);
        const int u = 2 * c + hh;
        return *reinterpret_cast<const bf16x8*>(&ks[krow * D + ((u ^ (krow % DC)) * 8)]);
    };

    // score and P tiles alternate between two register sets with the iteration parity
    floatx16 sA[QB][KB], sB[QB][KB];
    bf16x8 pA[QB][2 * KB], pB[QB][2 * KB];

    auto mfma_pv = [&](int i, const bf16x8& av, const bf16x8 (&pf)[QB][2 * KB]) {
        const int t = i / NOB, ob = i % NOB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            oacc[qb][ob] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[qb][t], oacc[qb][ob], 0, 0, 0);
    };
    auto mfma_qk = [&](int i, const bf16x8& av, floatx16 (&s)[QB][KB]) {
        const int c = i / KB, kb = i % KB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (c == 0) {
                const floatx16 zero = {};
                s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[qb][c], zero, 0, 0, 0);
            } else {
                s[qb][kb] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[qb][c], s[qb][kb], 0, 0, 0);
            }
        }
    };
    auto pv_all = [&](const __bf16* vs, const bf16x8 (&pf)[QB][2 * KB]) {
#pragma unroll
        for (int i = 0; i < NPV; ++i) mfma_pv(i, pv_operand(vs, i), pf);
    };
    auto qk_all = [&](const __bf16* ks, floatx16 (&s)[QB][KB]) {
#pragma unroll
        for (int i = 0; i < NQK; ++i) mfma_qk(i, qk_operand(ks, i), s);
    };

    // ---- softmax pieces
    auto row_max = [&](floatx16 (&s)[QB][KB], int qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s[qb][kb][a]);
        return wave_halves_max(mx) * c2;
    };
    // numerators of a pair of elements: k = ((qb * KB + kb) * 2 + u) * 4 + e covers
    // accumulator slots 8u + 2e and 8u + 2e + 1 of block (qb, kb)
    constexpr int NEXP = QB * KB * 8;
    auto exp_pair = [&](floatx16 (&s)[QB][KB], bf16x8 (&pf)[QB][2 * KB], int k,
                        const float (&nm)[QB], float (&sum)[QB]) {
        const int e = k % 4, u = (k / 4) % 2, kb = (k / 8) % KB, qb = k / (8 * KB);
        floatx2 pr = {fast_exp2(fmaf(s[qb][kb][8 * u + 2 * e], c2, nm[qb])),
                      fast_exp2(fmaf(s[qb][kb][8 * u + 2 * e + 1], c2, nm[qb]))};
        bf16x2 pb = __builtin_convertvector(pr, bf16x2);
        // keep the numerators at this point of the schedule (no sinking past the fences)
        uint32_t pbits = __builtin_bit_cast(uint32_t, pb);
        asm volatile("" : "+v"(pbits));
        pb = __builtin_bit_cast(bf16x2, pbits);
        // the row sum takes the same bf16 numerators that enter P V
        sum[qb] = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(__bf16)1.f, (__bf16)1.f}, sum[qb],
                                                  false);
        asm volatile("" : "+v"(sum[qb]));
        pf[qb][2 * kb + u][2 * e] = pb[0];
        pf[qb][2 * kb + u][2 * e + 1] = pb[1];
    };
    auto mask_tail = [&](floatx16 (&s)[QB][KB], int kt) {
        const int k0 = tile_k0(kt);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int key = k0 + kb * 32 + 16 * (a / 8) + 8 * hh + (a % 8);
                    if (key >= kend) s[qb][kb][a] = -INFINITY;
                }
    };

    // prologue: K_0, K_1 -> LDS; S_0; (register path) stage K_2 and V_0
    if constexpr (DMA) {
        dma_k(0, sk0);
        dma_k(1, sk1);
        dma_wait();
    } else {
        load_k(0);
        store_k(sk0);
        load_k(1);
        store_k(sk1);
    }
    __syncthreads();
    qk_all(sk0, sA);
    if constexpr (GV) {
        load_k(min(2, nkt - 1));
        // V_0 token-major before the first barrier; V_1 staged for iteration 0
        load_v(0);
        store_v(st0);
        load_v(min(1, nkt - 1));
    }

    // iteration j: softmax(S_j) || P_{j-1} V_{j-1} and Q K_{j+1}^T; loads V_j, K_{j+2}
    auto iteration = [&](int j, auto parity_tag, auto has_pv_tag, auto has_qk_tag) {
        constexpr int P = decltype(parity_tag)::value;
        constexpr bool HAS_PV = decltype(has_pv_tag)::value;
        constexpr bool HAS_QK = decltype(has_qk_tag)::value;
        __bf16* const my_k = P ? sk1 : sk0;       // K_{j+2} goes here (held K_j)
        __bf16* const my_v = P ? sv1 : sv0;       // V_j goes here (held V_{j-2})
        const __bf16* const rd_k = P ? sk0 : sk1; // holds K_{j+1}
        const __bf16* const rd_v = P ? sv0 : sv1; // holds V_{j-1}
        floatx16 (&s_in)[QB][KB] = P ? sB : sA;    // S_j
        floatx16 (&s_out)[QB][KB] = P ? sA : sB;   // S_{j+1}
        bf16x8 (&p_out)[QB][2 * KB] = P ? pB : pA; // P_j
        bf16x8 (&p_in)[QB][2 * KB] = P ? pA : pB;  // P_{j-1}
        // only the first tile (when it is also the last) and the last can reach kend
        if ((!HAS_QK || !HAS_PV) && tile_k0(j) + BC > kend) mask_tail(s_in, j);
        dma_wait();
        __syncthreads();
        // DMA: K_{j+2} and V_j go straight to the slots freed by the barrier and land
        // before the next one.  GATHER = 1: the staged K_{j+2} goes there, then K_{j+3} is
        // staged (indices past the end reload the last tile, unused); V_{j+1} goes
        // token-major into the free staging slot and V_j (staged last iteration) is read
        // transposed now, then written to the V^T slot during the steps
        uint4 vtr = {};
        if constexpr (DMA) {
            if (HAS_QK && j + 2 < nkt) dma_k(j + 2, my_k);
            dma_v(j, my_v);
        } else {
            if (HAS_QK) store_k(my_k);
            store_v(P ? st0 : st1);
            vtr = transpose_read(P ? st1 : st0);
            if (HAS_QK) load_k(min(j + 3, nkt - 1));
            load_v(min(j + 2, nkt - 1));
        }

        // SPARSE: a wave skips the products and numerators of tiles its query block does not
        // see (their weights are zero; scores left stale are never read: see check)
        const bool pv_on = !SPARSE || !HAS_PV || tile_on(j - 1);
        const bool qk_on = !SPARSE || !HAS_QK || tile_on(j + 1);
        const bool sm_on = !SPARSE || tile_on(j);
        constexpr int S0 = HAS_PV ? 0 : NPV;           // first MFMA step
        constexpr int S1 = HAS_QK ? NPV + NQK : NPV;   // one past the last step
        constexpr int NST = S1 - S0;
        // operand reads run this far ahead (measured best per load path)
        constexpr int LEAD = DMA ? FWD_LEAD : FWD_LEAD_GATHER;
        // Offset update.  Each lane first takes the maximum of its own scores only; the
        // wave raises m (exact maximum over both lane halves, rescale of l now and of O
        // after this iteration's P V products) only if some lane's maximum exceeds m by
        // more than kLazy -- a uniform branch that is rarely taken after the first tile.
        constexpr int FIRST = QB;                      // steps before the numerators start
        float nm[QB], alpha[QB];
        bool grow[QB];
        auto check = [&](int qb) {
            if constexpr (SPARSE) {
                if (!tile_on(j)) {                     // wave-uniform: zero weight
                    grow[qb] = false;
                    alpha[qb] = 1.f;
                    nm[qb] = -INFINITY;
                    return;
                }
            }
            float mx = s_in[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int a = 0; a < 16; ++a) mx = fmaxf(mx, s_in[qb][kb][a]);
            grow[qb] = __ballot(mx * c2 > m[qb] + kLazy) != 0;   // wave-uniform
            alpha[qb] = 1.f;
            if (grow[qb]) {
                asm volatile("");
                const float mrow = wave_halves_max(mx) * c2;
                const float m_new = fmaxf(m[qb], mrow);
                alpha[qb] = fast_exp2(m[qb] - m_new);
                m[qb] = m_new;
                l[qb] *= alpha[qb];
            }
            nm[qb] = -m[qb];
        };
        // step order: with both products present, PV and QK steps alternate so that
        // each dependent QK accumulation is separated by an independent PV MFMA
        auto step_id = [&](int k) -> int {       // returns a PV index (< NPV) or NPV + QK index
            if constexpr (HAS_PV && HAS_QK) {
                if constexpr (NPV == NQK) return (k & 1) ? NPV + (k >> 1) : (k >> 1);
            }
            return S0 + k;
        };
        auto load_op = [&](int st) -> bf16x8 {
            return st < NPV ? pv_operand(rd_v, st) : qk_operand(rd_k, st - NPV);
        };
        static_assert(NST > FIRST, "every iteration has products to overlap");
        {
            bf16x8 opnd[LEAD + 1];
#pragma unroll
            for (int k = 0; k < LEAD; ++k) opnd[k] = load_op(step_id(k));
#pragma unroll
            for (int k = 0; k < NST; ++k) {
                const int st = step_id(k);
                if (k + LEAD < NST) opnd[(k + LEAD) % (LEAD + 1)] = load_op(step_id(k + LEAD));
                if (st < NPV) {
                    if (pv_on) mfma_pv(st, opnd[k % (LEAD + 1)], p_in);
                } else {
                    if (qk_on) mfma_qk(st - NPV, opnd[k % (LEAD + 1)], s_out);
                }
                if (GV && k == (NST > FWD_TW ? FWD_TW : NST - 1)) transpose_write(vtr, my_v);
                // softmax slice: offset check first, then numerators
                if (k < QB) check(k);
                if (k >= FIRST && sm_on) {
                    const int lo = (k - FIRST) * NEXP / (NST - FIRST);
                    const int hi = (k - FIRST + 1) * NEXP / (NST - FIRST);
#pragma unroll
                    for (int e = lo; e < hi; ++e) exp_pair(s_in, p_out, e, nm, l);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // O holds P_{j-1} V_{j-1} in the old scale: rescale after those products
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            if (grow[qb]) {
                asm volatile("");
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                    for (int a = 0; a < 16; ++a) oacc[qb][ob][a] *= alpha[qb];
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
        __bf16* const vs = (jl & 1) ? sv1 : sv0;
        dma_wait();
        __syncthreads();
        if (!SPARSE || tile_on(jl)) {              // (SPARSE: skipped tiles left P stale)
            if (jl & 1) pv_all(vs, pB);
            else pv_all(vs, pA);
        }
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = wave_halves_sum(l[qb]);
        // (SPARSE rows that see no key: l = 0, O = 0, lse = -inf)
        const float inv = (SPARSE && l_tot == 0.f) ? 0.f : 1.f / l_tot;
        const int q_row = q_base + 32 * qb;
        if (PARTIAL && part_wg) {
            if (q_row < N) {
                const int64_t part = (int64_t)(unit - n_full) * n_split + split;
                const int64_t r = part * BR + (q_row - qt * BR);
                float* orow = OP + r * D;
#pragma unroll
                for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<floatx4*>(orow + ob * 32 + j * 8 + hh * 4) =
                            floatx4{oacc[qb][ob][4 * j] * inv, oacc[qb][ob][4 * j + 1] * inv,
                                    oacc[qb][ob][4 * j + 2] * inv, oacc[qb][ob][4 * j + 3] * inv};
                if (hh == 0) LP[r] = (m[qb] + log2f(l_tot)) * kLn2;
            }
            continue;
        }
        if (q_row < N) {
            __bf16* orow = O + (((int64_t)b * N + q_row) * H + h) * D;
#pragma unroll
            for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    floatx4 v = {oacc[qb][ob][4 * j] * inv, oacc[qb][ob][4 * j + 1] * inv,
                                 oacc[qb][ob][4 * j + 2] * inv, oacc[qb][ob][4 * j + 3] * inv};
                    *reinterpret_cast<bf16x4*>(orow + ob * 32 + j * 8 + hh * 4) =
                        __builtin_convertvector(v, bf16x4);
                }
            if (LSE != nullptr && hh == 0)
                LSE[(int64_t)bh * N + q_row] =
                    (SPARSE && l_tot == 0.f) ? -INFINITY : (m[qb] + log2f(l_tot)) * kLn2;
        }
    }
}

template <int D, int NW, int QB, int BC, int GATHER, bool SPARSE = false>
hipError_t launch_d(const void* q, const void* k, const void* vt, const StreamTable& st, int B,
                    int H, int N, int64_t ldv, float softmax_scale, void* o, float* lse,
                    hipStream_t stream, const uint8_t* mask = nullptr,
                    const int32_t* order = nullptr) {
    constexpr int BR = NW * QB * 32;
    const int n_qtiles = (N + BR - 1) / BR;
    const int total = n_qtiles * B * H;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QB, BC, GATHER, SPARSE>), dim3(total),
                       dim3(NW * 64), 0, stream, static_cast<const __bf16*>(q),
                       static_cast<const __bf16*>(k), static_cast<const __bf16*>(vt), st, mask, H,
                       N, ldv, softmax_scale * kLog2e, static_cast<__bf16*>(o), lse, n_qtiles,
                       total, 1, nullptr, nullptr, 0, order);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* vt, int B, int H, int N,
                           int D, int64_t ldv, float softmax_scale, void* o, float* lse,
                           hipStream_t stream) {
    // head size 64 (4 KB tiles) keeps 4 waves so that each wave still moves whole 1 KB loads
    const StreamTable none{};
    return D == 64 ? launch_d<64, 4, FWD_QB, FWD_BC, 0>(q, k, vt, none, B, H, N, ldv,
                                                            softmax_scale, o, lse, stream)
                   : launch_d<128, FWD_NW, FWD_QB, FWD_BC, 0>(q, k, vt, none, B, H, N, ldv,
                                                                  softmax_scale, o, lse, stream);
}

hipError_t launch_fwd_bf16_sparse(const void* q, const void* k, const void* vt,
                                  const uint8_t* mask, int B, int H, int N, int D, int64_t ldv,
                                  float softmax_scale, void* o, float* lse, hipStream_t stream,
                                  const int32_t* plan) {
    // a plan entry names one workgroup: both head sizes run 128-row workgroups
    static_assert(FWD_NW_SPARSE * FWD_QB * 32 == JA_SPARSE_BLOCK && 4 * FWD_QB * 32 == JA_SPARSE_BLOCK,
                  "one workgroup per query block of the mask");
    const StreamTable none{};
    return D == 64 ? launch_d<64, 4, FWD_QB, FWD_BC, 0, true>(q, k, vt, none, B, H, N, ldv,
                                                                  softmax_scale, o, lse, stream,
                                                                  mask, plan)
                   : launch_d<128, FWD_NW_SPARSE, FWD_QB, FWD_BC, 0, true>(
                         q, k, vt, none, B, H, N, ldv, softmax_scale, o, lse, stream, mask, plan);
}

namespace {

// ---- dispatch plan of the block-sparse forward.  Workgroup position p (after xcd_remap)
//      runs on XCD x for p in that XCD's share [c0, c0 + n) of the positions, in
//      increasing p.  A query block whose mask row allows more than twice its share's mean
//      number of key blocks (the text rows of a joint sequence see every block) is moved
//      to the front of its share, the others keep their order: the long workgroups then
//      start first instead of trailing the last (b, h) of a share, while consecutive
//      short ones still share their (b, h)'s keys in L2.

// pass 1: number of allowed key blocks of each query block (one wave per mask row)
__global__ __launch_bounds__(256) void sparse_plan_count_kernel(const uint8_t* __restrict__ MASK,
                                                                int nb, int total,
                                                                int32_t* __restrict__ CNT) {
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (u >= total) return;                      // wave-uniform
    const uint8_t* row = MASK + (int64_t)u * nb;
    int c = 0;
    for (int base = 0; base < nb; base += 64) {
        const int j = base + lane;
        c += __popcll(__ballot(j < nb && row[j] != 0));
    }
    if (lane == 0) CNT[u] = c;
}

// pass 2: one workgroup per XCD share turns the counts (in PLAN) into the order, in place
__global__ __launch_bounds__(1024) void sparse_plan_order_kernel(int total,
                                                                 int32_t* __restrict__ PLAN) {
    __shared__ uint32_t longbit[JA_SPARSE_PLAN_MAX / 8 / 32];
    __shared__ long long wsum[16];
    __shared__ int wlong[16];
    const int x = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = total >> 3, r = total & 7;     // the shares of xcd_remap
    const int c0 = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    const int n = q + (x < r ? 1 : 0);
    // each wave owns a segment of whole 64-entry steps
    const int seg = (((n + 15) / 16) + 63) / 64 * 64;
    const int s0 = min(n, wv * seg), s1 = min(n, s0 + seg);
    int32_t* P = PLAN + c0;
    long long sum = 0;
    for (int i = s0 + lane; i < s1; i += 64) sum += P[i];
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) wsum[wv] = sum;
    __syncthreads();
    long long all = 0;
    for (int v = 0; v < 16; ++v) all += wsum[v];
    // flags: count * n > 2 * (sum of the share's counts), i.e. above twice the mean
    int nl = 0;
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        const bool lg = i < s1 && (long long)P[i] * n > 2 * all;
        const uint64_t bl = __ballot(lg);
        nl += __popcll(bl);
        if (lg) atomicOr(&longbit[i >> 5], 1u << (i & 31));
        else if (i < s1) atomicAnd(&longbit[i >> 5], ~(1u << (i & 31)));
    }
    if (lane == 0) wlong[wv] = nl;
    __syncthreads();                             // every count is read before any is overwritten
    int pl = 0, n_long = 0;
    for (int v = 0; v < 16; ++v) {
        pl += v < wv ? wlong[v] : 0;
        n_long += wlong[v];
    }
    int ps = n_long + (s0 - pl);                 // short entries before this segment
    for (int base = s0; base < s1; base += 64) {
        const int i = base + lane;
        const bool in = i < s1;
        const bool lg = in && ((longbit[i >> 5] >> (i & 31)) & 1u);
        const uint64_t bl = __ballot(lg), bs = __ballot(in && !lg);
        const uint32_t below_l = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(bl >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bl, 0u));
        const uint32_t below_s = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0u));
        if (in) P[lg ? pl + (int)below_l : ps + (int)below_s] = c0 + i;
        pl += __popcll(bl);
        ps += __popcll(bs);
    }
}

}  // namespace

hipError_t launch_sparse_plan(const uint8_t* mask, int units, int nb, int32_t* plan,
                              hipStream_t stream) {
    hipLaunchKernelGGL(sparse_plan_count_kernel, dim3((units + 3) / 4), dim3(256), 0, stream,
                       mask, nb, units, plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sparse_plan_order_kernel, dim3(8), dim3(1024), 0, stream, units, plan);
    return hipGetLastError();
}

int splitkv_slots(int D) {
    // workgroups that run at once: one per CU for the 8-wave D = 128 kernel, as the
    // runtime's occupancy calculation gives for the kernel actually launched
    int dev = 0, cus = 256, per = 1;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    hipError_t e = D == 64
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &per, fwd_bf16_kernel<64, 4, FWD_QB, FWD_BC, 0, false, true>, 4 * 64, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &per, fwd_bf16_kernel<128, FWD_NW, FWD_QB, FWD_BC, 0, false, true>, FWD_NW * 64,
              0);
    if (e != hipSuccess || per < 1) per = 1;
    return cus * per;
}

int splitkv_rows_per_tile(int D) { return D == 64 ? 4 * FWD_QB * 32 : FWD_NW * FWD_QB * 32; }

namespace {
// split-KV launch for gather mode G (0: packed Q, K, V^T; 1: all three from the streams;
// 2: Q and K from the streams, V^T packed): the split kernel and the merge, or the plain
// forward when nothing is split
template <int G>
hipError_t launch_splitkv_mode(const void* q, const void* k, const void* vt,
                               const StreamTable& st, int B, int H, int N, int D, int64_t ldv,
                               float softmax_scale, int n_split, int slots, float* o_part,
                               float* lse_part, void* o, float* lse, hipStream_t stream) {
    const int tiles = (N + FWD_BC - 1) / FWD_BC;
    n_split = n_split < tiles ? n_split : tiles;               // every key range non-empty
    const int BRr = splitkv_rows_per_tile(D);
    const int n_units = (N + BRr - 1) / BRr * B * H;
    const int tail = n_units % slots;                         // tiles of the last, partial round
    if (n_split <= 1 || tail == 0)
        return D == 64 ? launch_d<64, 4, FWD_QB, FWD_BC, G>(q, k, vt, st, B, H, N, ldv,
                                                            softmax_scale, o, lse, stream)
                       : launch_d<128, FWD_NW, FWD_QB, FWD_BC, G>(q, k, vt, st, B, H, N, ldv,
                                                                  softmax_scale, o, lse, stream);
    const int n_full = n_units - tail;
    auto go = [&](auto d_tag, auto nw_tag) -> hipError_t {
        constexpr int DD = decltype(d_tag)::value, NWW = decltype(nw_tag)::value;
        constexpr int BR = NWW * FWD_QB * 32;
        constexpr int RPB = 256 / (DD / 4);
        const int n_qtiles = (N + BR - 1) / BR;
        const int total = n_full + tail * n_split;
        hipLaunchKernelGGL((fwd_bf16_kernel<DD, NWW, FWD_QB, FWD_BC, G, false, true>),
                           dim3(total), dim3(NWW * 64), 0, stream, static_cast<const __bf16*>(q),
                           static_cast<const __bf16*>(k), static_cast<const __bf16*>(vt), st,
                           nullptr, H, N, ldv, softmax_scale * kLog2e, static_cast<__bf16*>(o),
                           lse, n_qtiles, total, n_split, o_part, lse_part, n_full);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((splitkv_merge_kernel<DD, BR>), dim3(tail * (BR / RPB)), dim3(256), 0,
                           stream, o_part, lse_part, n_split, n_full, n_qtiles, H, N,
                           static_cast<__bf16*>(o), lse);
        return hipGetLastError();
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using I4 = std::integral_constant<int, 4>;
    using INW = std::integral_constant<int, FWD_NW>;
    return D == 64 ? go(I64{}, I4{}) : go(I128{}, INW{});
}
}  // namespace

hipError_t launch_fwd_bf16_splitkv(const void* q, const void* k, const void* vt, int B, int H,
                                   int N, int D, int64_t ldv, float softmax_scale, int n_split,
                                   int slots, float* o_part, float* lse_part, void* o,
                                   float* lse, hipStream_t stream) {
    const StreamTable none{};
    return launch_splitkv_mode<0>(q, k, vt, none, B, H, N, D, ldv, softmax_scale, n_split, slots,
                                  o_part, lse_part, o, lse, stream);
}

hipError_t launch_fwd_bf16_streams_splitkv(const StreamTable& st, const void* vt, int64_t ldv,
                                           int B, int H, int N, int D, float softmax_scale,
                                           int n_split, int slots, float* o_part,
                                           float* lse_part, void* o, float* lse,
                                           hipStream_t stream) {
    return vt == nullptr
        ? launch_splitkv_mode<1>(nullptr, nullptr, nullptr, st, B, H, N, D, 0, softmax_scale,
                                 n_split, slots, o_part, lse_part, o, lse, stream)
        : launch_splitkv_mode<2>(nullptr, nullptr, vt, st, B, H, N, D, ldv, softmax_scale,
                                 n_split, slots, o_part, lse_part, o, lse, stream);
}

// ---- allocation-free split-KV: the partial outputs and log-sum-exps live in this
//      file-scope device array instead of a caller workspace.  Every device the library
//      runs on holds its own copy (until the process ends) at its own address, looked up
//      once per device with that device current; host code passes that address to the
//      kernels, never the array's name (whose host-side value is only a stand-in).
namespace {
static __device__ __align__(256) float scratch[JA_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

hipError_t launch_fwd_bf16_splitkv_noalloc(const void* q, const void* k, const void* vt, int B,
                                           int H, int N, int D, int64_t ldv, float softmax_scale,
                                           int n_split, int slots, int64_t parts, void* o,
                                           float* lse, hipStream_t stream) {
    // parts = split tiles x key ranges, checked by the caller against JA_SCRATCH_BYTES:
    // O partials [parts][rows][D], then lse partials [parts][rows]
    void* base = nullptr;
    if (parts > 0) {
        const hipError_t e = scratch_address(&base);
        if (e != hipSuccess) return e;
    }
    float* o_part = static_cast<float*>(base);
    float* lse_part = parts > 0 ? o_part + parts * splitkv_rows_per_tile(D) * D : nullptr;
    return launch_fwd_bf16_splitkv(q, k, vt, B, H, N, D, ldv, softmax_scale, n_split, slots,
                                   o_part, lse_part, o, lse, stream);
}

hipError_t launch_fwd_bf16_streams(const StreamTable& st, int B, int H, int N, int D,
                                   float softmax_scale, void* o, float* lse,
                                   hipStream_t stream) {
    return D == 64 ? launch_d<64, 4, FWD_QB, FWD_BC, 1>(nullptr, nullptr, nullptr, st, B, H, N,
                                                        0, softmax_scale, o, lse, stream)
                   : launch_d<128, FWD_NW, FWD_QB, FWD_BC, 1>(nullptr, nullptr, nullptr, st, B,
                                                              H, N, 0, softmax_scale, o, lse,
                                                              stream);
}

}  // namespace ja

// moe_expert_ffn_fused / moe_expert_ffn_fp8_fused: the expert FFN of every
// group as ONE kernel in which the intermediate h never leaves the CU.
//
// The fused FC1+FC2 form is the one the TensorRT-LLM page lists as its
// CuteDslFc12 backend (section "后端的三种形态与两个调度器家族": FC1 and FC2 in
// one kernel, the intermediate kept on chip).  Here a work item is one tile
// of BM rows of one group; its workgroup
//   phase 1: computes h[BM, I] = silu(x W1^T) * (x W3^T) in 2I/BN column
//            sub-tiles (each a K = H loop over the gathered activation rows
//            and the expert's w13 rows) and writes every sub-tile's h into an
//            LDS buffer that holds all I columns of the BM rows: bf16, or for
//            fp8 activations e4m3 codes plus one fp32 scale per row and 128
//            channels, quantised exactly as the two-call path quantises them;
//   phase 2: computes out[BM, H] = h W2^T in ceil(H/BN) column sub-tiles, a
//            K = I loop that reads its activation fragments from that LDS
//            buffer and streams only the expert's w2 rows.
// The arithmetic per output element (operands, MFMA forms, K order, block
// scaling, rounding of h) is the one of moe_expert_ffn / moe_expert_ffn_fp8,
// so the results are bit-identical to the two-call path.
//
// Parallelism.  A group of n rows has ceil(n/BM) row tiles; each tile can be
// split over `nsplit` workgroups, which all compute the tile's h (phase 1 is
// repeated) and divide its FC2 column sub-tiles round-robin.  The work list
// (group, row tile, split) is built on the device from the offsets, items of
// one group are adjacent, and the persistent grid walks it with the same
// XCD-aware mapping as the two-call kernels, so the workgroups that read one
// expert's weights run on one XCD and share its L2.
//
// Transfers use the direct-to-LDS ring of the two-call engine (dma.h): each
// stage is one K slice; a sub-tile's first S-1 slices are issued before the
// previous sub-tile's epilogue.  The ring, h and the tables fill one CU's LDS
// (about 140 KB), so one workgroup of 4 waves runs per CU.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "dma.h"

namespace moe {
namespace {

struct FusedArgs {
    const char* x;          // bf16 x [T, H], or e4m3 codes xq [T, H]
    const float* xscale;    // fp8 activations: [T, H/128]
    const char* w13;        // [G, 2I, H]
    const float* w13s;      // fp8 weights: [G, 2I/128, H/128]
    const char* w2;         // [G, H, I]
    const float* w2s;       // fp8 weights: [G, H/128, I/128]
    char* out;              // bf16 fc2_out [R, H]
    const int32_t* offsets;
    const int32_t* permuted_pair;
    int T, k, E, G, H, I;
    int nsplit;             // workgroups per row tile, 1 <= nsplit <= ceil(H/BN)
};

// BM rows per tile (one wave row: every wave holds all BM rows), BN columns
// per sub-tile over WN waves, a ring of S stages; W8: fp8 weights; A8: fp8
// activations (and weights); HROW: the largest h row in bytes the LDS buffer
// holds (I * bytes per h element).
template <int BM_, int BN_, int WN_, int S_, bool W8_, bool A8_, int HROW_>
struct FusedCfg {
    static constexpr int BM = BM_, BN = BN_, WN = WN_, S = S_;
    static constexpr int NW = WN, NT = 64 * WN;
    static constexpr bool A8 = A8_;
    static constexpr bool W8 = W8_ || A8_;
    static constexpr bool WNARROW = W8 && !A8;             // fp8 weights widened to bf16
    static constexpr int BK = A8 ? 128 : 64;               // K per stage
    static constexpr int KSTEPS = A8 ? 1 : BK / 32;
    static constexpr int BROWB = WNARROW ? 64 : 128;       // weight bytes per staged row
    static constexpr int A_OPS = BM / 8;                   // 1 KB transfers per stage: activations
    static constexpr int B_OPS = BN * BROWB / 1024;        // ... weights
    static constexpr int NOPS1 = A_OPS + B_OPS, NOPS2 = B_OPS;
    static constexpr int Q1 = (NOPS1 + NW - 1) / NW;       // most 1 KB transfers of one wave
    static constexpr int Q2 = (NOPS2 + NW - 1) / NW;
    static constexpr int QS = A8 ? 1 : 0;                  // + the activation-scale transfer
    static constexpr int QMAX = Q1 + QS;
    static constexpr int A_BYTES = BM * 128;
    static constexpr int B_BYTES = BN * BROWB;
    static constexpr int SA_BYTES = A8 ? NW * 256 : 0;     // per-wave activation-scale slots
    static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
    static constexpr int WTN = BN / WN;
    static constexpr int MI = BM / 16, NI = WTN / 16;
    static constexpr int HROW = HROW_;
    static constexpr int HPITCH = HROW + 128;              // odd multiple of 128 B: the ring's bank pattern
    static constexpr int HSN = A8 ? HROW / 128 : 1;        // h scales per row
    static constexpr int LDS_BYTES = S * STAGE + BM * HPITCH + BM * HSN * 4 + BM * WN * 4 +
                                     2 * (kMaxGroups + 1) * 4;
    static_assert(BM % 16 == 0 && BM <= 64, "row tile");
    static_assert(WTN % 32 == 0, "a wave holds whole gate/up column pairs");
    static_assert(!A8 || BN == 256, "A8: one FC1 sub-tile = one 128-channel block of h");
    static_assert(B_OPS % NW == 0, "phase-2 transfers split evenly");
    static_assert(HROW % 128 == 0 && (HPITCH / 128) % 2 == 1, "h row: an odd number of 128-byte units");
    static_assert(S >= 2 && S <= 8 && LDS_BYTES <= 160 * 1024, "LDS");
};

template <class C>
__global__ __launch_bounds__(C::NT) void fused_ffn_kernel(FusedArgs a)
{
    __shared__ __attribute__((aligned(1024))) char lds[C::S * C::STAGE];
    __shared__ __attribute__((aligned(16))) char hbuf[C::BM * C::HPITCH];
    __shared__ float hsc[C::BM * C::HSN];    // A8: h scales [BM][I/128]
    __shared__ float s_amax[C::BM * C::WN];  // A8: row maxima per wave
    __shared__ int s_off[kMaxGroups + 1];
    __shared__ int s_item0[kMaxGroups + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave;
    const int G = a.G, ns = a.nsplit;
    const int N1 = 2 * a.I / C::BN;                // FC1 sub-tiles
    const int N2 = (a.H + C::BN - 1) / C::BN;      // FC2 sub-tiles
    const int nk1 = a.H / C::BK, nk2 = a.I / C::BK;

    // ---- work list: group g owns ceil(n / BM) * nsplit consecutive items
    for (int g = tid; g <= G; g += C::NT) s_off[g] = a.offsets[g];
    __syncthreads();
    if (wave == 0) {
        const int per = (G + 63) / 64;
        const int g0 = lane * per, g1 = min(G, g0 + per);
        auto nitems = [&](int g) { return (s_off[g + 1] - s_off[g] + C::BM - 1) / C::BM * ns; };
        int sum = 0;
        for (int g = g0; g < g1; ++g) sum += nitems(g);
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        int run = incl - sum;
        for (int g = g0; g < g1; ++g) {
            s_item0[g] = run;
            run += nitems(g);
        }
        if (lane == 63) s_item0[G] = incl;
    }
    __syncthreads();
    const int total = s_item0[G];
    const int nb = gridDim.x;
    const int slot = (nb % 8) == 0 ? (blockIdx.x >> 3) + (blockIdx.x & 7) * (nb >> 3) : blockIdx.x;
    int item = slot;
    if (item >= total) return;

    struct Item {
        int g, row0, nrows, m0, split;
    };
    auto decode = [&](int it) {
        int lo = 0, hi = G - 1;
        while (lo < hi) {  // last g with s_item0[g] <= it
            const int mid = (lo + hi + 1) >> 1;
            if (__builtin_amdgcn_readfirstlane(s_item0[mid]) <= it) lo = mid; else hi = mid - 1;
        }
        Item r;
        r.g = lo;
        r.row0 = __builtin_amdgcn_readfirstlane(s_off[lo]);
        r.nrows = __builtin_amdgcn_readfirstlane(s_off[lo + 1]) - r.row0;
        const int local = it - __builtin_amdgcn_readfirstlane(s_item0[lo]);
        r.m0 = (local / ns) * C::BM;
        r.split = local % ns;
        return r;
    };

    const size_t x_ld = (size_t)a.H * (C::A8 ? 1 : 2);
    const size_t w1_ld = (size_t)a.H * (C::W8 ? 1 : 2), w2_ld = (size_t)a.I * (C::W8 ? 1 : 2);
    const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)lds;

    // Transfer o = q*NW + wave of a stage (q < Q1 in phase 1, < Q2 in phase 2).
    // Phase 1: o < A_OPS stages activation rows 8o .. 8o+7, the others weight
    // rows (8 of 128 bytes or 16 narrow rows of 64 bytes each); phase 2 stages
    // weight rows only, into the same place of the stage.  With fp8
    // activations every wave also stages the scales of the tile's rows
    // (q = Q1, lane l: row l % BM).  Lane l writes bytes [16l, 16l+16) of the
    // 1 KB: row l/8 (l/4 narrow), physical chunk l%8 (l%4).
    auto n_ops = [&](int nops) { return nops > wave ? (nops - wave + C::NW - 1) / C::NW : 0; };
    const int nw1 = n_ops(C::NOPS1) + C::QS, nw2 = n_ops(C::NOPS2);  // transfers of this wave per stage
    auto b_row = [&](int ob) { return C::WNARROW ? ob * 16 + (lane >> 2) : ob * 8 + (lane >> 3); };
    auto b_chunk = [&](int row) { return C::WNARROW ? (lane & 3) ^ ((row >> 2) & 3) : (lane & 7) ^ (row & 7); };
    const int s_row = lane % C::BM;

    // token of tile row rr of item `it` (padding rows: token 0), from the raw
    // permuted_pair entry fetched ahead
    auto pp_raw = [&](const Item& it, int rr) -> int {
        const int i = (it.g < a.E && rr < it.nrows) ? it.row0 + rr : 0;
        return *(const __attribute__((address_space(1))) int*)(a.permuted_pair + i);
    };
    auto token = [&](const Item& it, int rr, int raw) -> long {
        const int tok = (rr >= it.nrows) ? 0 : (it.g < a.E ? raw / a.k : rr);
        return tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
    };
    // raw entries this wave needs: A rows of its activation transfers, and the
    // scale row
    constexpr int NRAW = (C::A_OPS + C::NW - 1) / C::NW + C::QS;
    auto load_raw = [&](const Item& it, int (&raw)[NRAW]) {
#pragma unroll
        for (int q = 0; q < NRAW; ++q) {
            int rr;
            if (C::A8 && q == NRAW - 1) rr = it.m0 + s_row;
            else rr = it.m0 + (q * C::NW + wave) * 8 + (lane >> 3);
            raw[q] = (C::A8 && q == NRAW - 1) || q * C::NW + wave < C::A_OPS ? pp_raw(it, rr) : 0;
        }
    };
    // per-item byte offsets of the activation transfers and the scale transfer
    uint32_t aoff[NRAW];
    auto set_item = [&](const Item& it, const int (&raw)[NRAW]) {
#pragma unroll
        for (int q = 0; q < NRAW; ++q) {
            if (C::A8 && q == NRAW - 1) {
                aoff[q] = (uint32_t)(token(it, it.m0 + s_row, raw[q]) * (a.H / 128) * 4);
            } else {
                const int row = (q * C::NW + wave) * 8 + (lane >> 3);
                aoff[q] = (uint32_t)(token(it, it.m0 + row, raw[q]) * x_ld) + ((lane & 7) ^ (row & 7)) * 16;
            }
        }
    };

    const char* xbase = uniform_ptr(a.x);
    const char* sbase = uniform_ptr(reinterpret_cast<const char*>(a.xscale));
    const char* wbase;
    uint32_t src[C::QMAX];
    int ring = 0;  // ring slot of the current sub-tile's slice 0
    // source offsets of sub-tile (phase, nt) of item `it`
    auto set_sub = [&](const Item& it, bool p1, int nt) {
        if (p1) {
            wbase = uniform_ptr(a.w13 + (size_t)it.g * (2 * a.I) * w1_ld);
#pragma unroll
            for (int q = 0; q < C::Q1; ++q) {
                const int o = q * C::NW + wave;
                if (o < C::A_OPS) {
                    src[q] = aoff[q];
                } else {
                    const int j = b_row(o - C::A_OPS);
                    const int blk = j >> 4, pair = blk >> 1;
                    const int col = nt * (C::BN / 2) + pair * 16 + (j & 15);
                    const int wrow = (blk & 1) ? a.I + col : col;
                    src[q] = (uint32_t)(wrow * w1_ld) + b_chunk(j) * 16;
                }
            }
            if constexpr (C::A8) src[C::Q1] = aoff[NRAW - 1];
        } else {
            wbase = uniform_ptr(a.w2 + (size_t)it.g * a.H * w2_ld);
#pragma unroll
            for (int q = 0; q < C::Q2; ++q) {
                const int j = b_row(q * C::NW + wave);
                const int wrow = min(nt * C::BN + j, a.H - 1);  // partial last sub-tile
                src[q] = (uint32_t)(wrow * w2_ld) + b_chunk(j) * 16;
            }
        }
    };
    // transfers of K slice kt of the current sub-tile into ring slot st
    auto issue = [&](auto phase_tag, int st, int kt) {
        constexpr bool P1 = decltype(phase_tag)::value;
        const unsigned sb = lds_base + st * C::STAGE;
        if constexpr (P1) {
#pragma unroll
            for (int q = 0; q < C::Q1; ++q) {
                const int o = q * C::NW + wave;
                if (o < C::NOPS1)
                    dma16(__builtin_amdgcn_readfirstlane(sb + o * 1024), o < C::A_OPS ? xbase : wbase,
                          src[q] + (uint32_t)kt * (o < C::A_OPS ? 128u : (uint32_t)C::BROWB));
            }
            if constexpr (C::A8)
                dma4(__builtin_amdgcn_readfirstlane(sb + C::A_BYTES + C::B_BYTES + wave * 256), sbase,
                     src[C::Q1] + (uint32_t)kt * 4u);
        } else {
#pragma unroll
            for (int q = 0; q < C::Q2; ++q)
                dma16(__builtin_amdgcn_readfirstlane(sb + C::A_BYTES + (q * C::NW + wave) * 1024), wbase,
                      src[q] + (uint32_t)kt * (uint32_t)C::BROWB);
        }
    };
    // the first S-1 slices of a sub-tile (phase known only at run time)
    auto prologue = [&](bool p1, int nk) {
#pragma unroll
        for (int st = 0; st < C::S - 1; ++st) {
            if (st < nk) {
                if (p1) issue(std::true_type(), (ring + st) % C::S, st);
                else issue(std::false_type(), (ring + st) % C::S, st);
            }
        }
    };

    Item cur = decode(item);
    int raw[NRAW], nraw[NRAW];
    load_raw(cur, raw);
    set_item(cur, raw);
    int u = 0;                                      // sub-tile of the current item
    auto n_sub = [&](const Item& it) { return N1 + (N2 - it.split + ns - 1) / ns; };
    auto sub_nt = [&](const Item& it, int uu) { return uu < N1 ? uu : it.split + (uu - N1) * ns; };
    set_sub(cur, true, 0);
    prologue(true, nk1);
    Item nxt = cur;
    int next_item = item + nb;
    bool has_next_item = false;

    const int erow = lane & 15;        // result row within a 16x16 block
    const int ecol = (lane >> 4) * 4;  // first of its 4 columns
    const int g4 = lane >> 4;

    while (true) {
        const bool p1 = u < N1;
        const int nt = sub_nt(cur, u);
        const int nk = p1 ? nk1 : nk2;
        const int nwv = p1 ? nw1 : nw2;
        if (u == 0) {  // next item's token indices, consumed a whole item later
            next_item = item + nb;
            has_next_item = next_item < total;
            if (has_next_item) {
                nxt = decode(next_item);
                load_raw(nxt, nraw);
            }
        }

        f32x4_t acc[C::MI][C::NI];
        f32x4_t part[C::WNARROW ? C::MI : 1][C::WNARROW ? C::NI : 1];
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (C::WNARROW) {
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) part[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        // K loop of one sub-tile.  The activation operand comes from the ring
        // in phase 1 and from the h buffer in phase 2; everything else is
        // shared.
        auto kloop = [&](auto phase_tag) {
            constexpr bool P1 = decltype(phase_tag)::value;
            const int N = P1 ? 2 * a.I : a.H;   // weight rows of this GEMM
            const int K = P1 ? a.H : a.I;
            const float* wscale = P1 ? a.w13s : a.w2s;
            for (int kt = 0; kt < nk; ++kt) {
                wait_vmcnt_le<(C::S - 2) * C::QMAX>(min(C::S - 2, nk - 1 - kt) * nwv);
                lds_barrier();  // slice kt is in LDS for every wave; slot of slice kt-1 is free
                if (kt + C::S - 1 < nk) issue(phase_tag, (ring + kt + C::S - 1) % C::S, kt + C::S - 1);
                const char* la = lds + ((ring + kt) % C::S) * C::STAGE;
                const char* lb = la + C::A_BYTES;
                if constexpr (C::A8) {
                    const int sk = K / 128;
                    const __attribute__((address_space(4))) float* wsp =
                        (const __attribute__((address_space(4))) float*)wscale;
                    float sw0, sw1;
                    if (P1) {
                        const int col = nt * (C::BN / 2);  // the sub-tile's 128 h columns
                        sw0 = wsp[((size_t)cur.g * (N / 128) + col / 128) * sk + kt];
                        sw1 = wsp[((size_t)cur.g * (N / 128) + (a.I + col) / 128) * sk + kt];
                    } else {
                        const int wrow = min(nt * C::BN + wn * C::WTN, N - 1);
                        sw0 = sw1 = wsp[((size_t)cur.g * (N / 128) + wrow / 128) * sk + kt];
                    }
                    float s0[C::MI], s1[C::MI];
                    i32x8_t fa[C::MI];
#pragma unroll
                    for (int mi = 0; mi < C::MI; ++mi) {
                        const int row = mi * 16 + (lane & 15);
                        float sa;
                        if (P1) {
                            sa = reinterpret_cast<const float*>(lb + C::B_BYTES + wave * 256)[row];
                            fa[mi] = lds_row32(la, row, g4);
                        } else {
                            sa = hsc[row * C::HSN + kt];
                            // the K positions of lds_row32: chunks g4 and g4+4
                            const char* hr = hbuf + row * C::HPITCH + kt * 128;
                            const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(hr + ((g4 ^ (row & 7)) << 4));
                            const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(hr + (((g4 + 4) ^ (row & 7)) << 4));
                            fa[mi] = i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                                             (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
                        }
                        s0[mi] = sa * sw0;
                        s1[mi] = sa * sw1;
                    }
                    // MFMA j+1 is issued before the VALU that scales result j
                    constexpr int NB = C::MI * C::NI, LAGB = 2;
                    f32x4_t pr[LAGB + 1];
                    i32x8_t fb[2];
                    fb[0] = lds_row32(lb, wn * C::WTN + (lane & 15), g4);
#pragma unroll
                    for (int j = 0; j < NB + LAGB; ++j) {
                        if (j < NB) {
                            const int mi = j % C::MI, ni = j / C::MI;
                            if (mi == 0 && ni + 1 < C::NI)
                                fb[(ni + 1) & 1] = lds_row32(lb, wn * C::WTN + (ni + 1) * 16 + (lane & 15), g4);
                            pr[j % (LAGB + 1)] = mfma_fp8(fb[ni & 1], fa[mi]);
                        }
                        if (j >= LAGB) {
                            const int jj = j - LAGB, mi = jj % C::MI, ni = jj / C::MI;
                            acc[mi][ni] += ((P1 && (ni & 1)) ? s1[mi] : s0[mi]) * pr[jj % (LAGB + 1)];
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
#pragma unroll
                    for (int ks = 0; ks < C::KSTEPS; ++ks) {
                        const int kc = ks * 4 + (lane >> 4);
                        u32x4_t fa[C::MI], fb[C::NI];
#pragma unroll
                        for (int mi = 0; mi < C::MI; ++mi) {
                            const int row = mi * 16 + (lane & 15);
                            if (P1)
                                fa[mi] = *reinterpret_cast<const u32x4_t*>(la + dma_off(row, kc));
                            else
                                fa[mi] = *reinterpret_cast<const u32x4_t*>(hbuf + row * C::HPITCH + kt * 128 +
                                                                           ((kc ^ (row & 7)) << 4));
                        }
#pragma unroll
                        for (int ni = 0; ni < C::NI; ++ni) {
                            const int row = wn * C::WTN + ni * 16 + (lane & 15);
                            if constexpr (C::WNARROW) {
                                typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
                                const u32x2_t w = *reinterpret_cast<const u32x2_t*>(
                                    lb + dma_off_w8(row, ks * 2 + (lane >> 5)) + ((lane >> 4) & 1) * 8);
                                fb[ni] = fp8x8_to_bf16x8(w.x, w.y);
                            } else {
                                fb[ni] = *reinterpret_cast<const u32x4_t*>(lb + dma_off(row, kc));
                            }
                        }
#pragma unroll
                        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                            for (int ni = 0; ni < C::NI; ++ni) {
                                if constexpr (C::WNARROW) part[mi][ni] = mfma_frag(fb[ni], fa[mi], part[mi][ni], bf16_t());
                                else acc[mi][ni] = mfma_frag(fb[ni], fa[mi], acc[mi][ni], bf16_t());
                            }
                    }
                }
                if constexpr (C::WNARROW) {
                    if (kt & 1) {  // end of a 128-wide K block: acc += block scale * partial
                        const int kb = kt >> 1, sk = K / 128;
                        const __attribute__((address_space(4))) float* ws =
                            (const __attribute__((address_space(4))) float*)wscale;
#pragma unroll
                        for (int ni = 0; ni < C::NI; ++ni) {
                            const int j = wn * C::WTN + ni * 16;
                            int wrow;
                            if (P1) {
                                const int blk = j >> 4, pair = blk >> 1;
                                const int col = nt * (C::BN / 2) + pair * 16;
                                wrow = (blk & 1) ? a.I + col : col;
                            } else {
                                wrow = min(nt * C::BN + j, N - 1);
                            }
                            const float sc = ws[((size_t)cur.g * (N / 128) + wrow / 128) * sk + kb];
#pragma unroll
                            for (int mi = 0; mi < C::MI; ++mi) {
                                acc[mi][ni] += sc * part[mi][ni];
                                part[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                            }
                        }
                    }
                }
            }
        };
        if (p1) kloop(std::true_type());
        else kloop(std::false_type());

        // the next sub-tile's first slices go out before this one's epilogue
        lds_barrier();  // every wave is done reading the ring and, in phase 2, h
        const bool more_here = u + 1 < n_sub(cur);
        const bool has_next = more_here || has_next_item;
        if (has_next) {
            if (!more_here) set_item(nxt, nraw);
            const Item& nit = more_here ? cur : nxt;
            const int nu = more_here ? u + 1 : 0;
            set_sub(nit, nu < N1, sub_nt(nit, nu));
            ring = (ring + nk) % C::S;
            prologue(nu < N1, nu < N1 ? nk1 : nk2);
        }

        // Epilogue.  Lane l holds tile row l%16 of each 16-row block and four
        // consecutive columns 4*(l/16) + i of each 16-column block.
        if (p1) {
            if constexpr (C::A8) {
                // h -> e4m3 per row and 128 channels (the whole sub-tile); the
                // row maximum combines the 4 lanes and WN waves of a row
                float rmax[C::MI];
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi) {
                    rmax[mi] = 0.0f;
#pragma unroll
                    for (int q = 0; q < C::NI / 2; ++q) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float gt = acc[mi][2 * q][i];
                            const float up = acc[mi][2 * q + 1][i];
                            const float hv = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * up;
                            acc[mi][2 * q][i] = hv;
                            rmax[mi] = fmaxf(rmax[mi], fabsf(hv));
                        }
                    }
                    rmax[mi] = fmaxf(rmax[mi], __shfl_xor(rmax[mi], 16, 64));
                    rmax[mi] = fmaxf(rmax[mi], __shfl_xor(rmax[mi], 32, 64));
                    if (lane < 16) s_amax[(mi * 16 + erow) * C::WN + wn] = rmax[mi];
                }
                lds_barrier();
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi) {
                    const int row = mi * 16 + erow;
                    float amax = 0.0f;
#pragma unroll
                    for (int w = 0; w < C::WN; ++w) amax = fmaxf(amax, s_amax[row * C::WN + w]);
                    const float sc = amax / 448.0f;
#pragma unroll
                    for (int q = 0; q < C::NI / 2; ++q) {
                        const float hv[4] = {acc[mi][2 * q][0], acc[mi][2 * q][1], acc[mi][2 * q][2], acc[mi][2 * q][3]};
                        const int e = ((wn * C::WTN) / 32 + q) * 16 + ecol;  // channel within the block
                        *reinterpret_cast<uint32_t*>(hbuf + row * C::HPITCH + nt * 128 +
                                                     (((e >> 4) ^ (row & 7)) << 4) + (e & 15)) = fp8x4_code(hv, sc);
                    }
                    if (wn == 0 && lane < 16) hsc[row * C::HSN + nt] = sc;
                }
            } else {
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                    for (int q = 0; q < C::NI / 2; ++q) {
                        float hv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float gt = acc[mi][2 * q][i];
                            const float up = acc[mi][2 * q + 1][i];
                            hv[i] = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * up;
                        }
                        const int row = mi * 16 + erow;
                        const int c = nt * (C::BN / 2) + ((wn * C::WTN) / 32 + q) * 16 + ecol;  // h column
                        const int e = c & 63;  // within its 64-column K slice
                        typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
                        *reinterpret_cast<u32x2_t*>(hbuf + row * C::HPITCH + (c >> 6) * 128 +
                                                    (((e >> 3) ^ (row & 7)) << 4) + (e & 7) * 2) =
                            u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
                    }
            }
        } else {
            // FC2 rows staged 16 at a time per wave in the ring slot that the
            // next sub-tile fills last, then written as 16-byte column chunks
            // (non-temporal: fc2_out is read once, by the finalize)
            bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
            constexpr int PITCH = C::WTN * 2 + 16;
            constexpr int CPR = C::WTN / 8;
            constexpr int RPI = 64 / CPR;
            static_assert(16 * PITCH <= C::STAGE / C::NW && 16 % RPI == 0, "epilogue staging");
            const int fslot = has_next ? (ring + C::S - 1) % C::S : 0;
            char* stg = lds + fslot * C::STAGE + wave * (C::STAGE / C::NW);
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<u32x2_t*>(stg + erow * PITCH + (ni * 16 + ecol) * 2) =
                        u32x2_t{pack_bf16x2(acc[mi][ni][0], acc[mi][ni][1]), pack_bf16x2(acc[mi][ni][2], acc[mi][ni][3])};
                }
#pragma unroll
                for (int j = 0; j < 16 / RPI; ++j) {
                    const int r = j * RPI + lane / CPR, c = lane % CPR;
                    const u32x4_t d = *reinterpret_cast<const u32x4_t*>(stg + r * PITCH + c * 16);
                    const int rr = cur.m0 + mi * 16 + r;
                    const int col = nt * C::BN + wn * C::WTN + c * 8;
                    if (rr < cur.nrows && col < a.H)
                        __builtin_nontemporal_store(d, (__attribute__((address_space(1))) u32x4_t*)(out + (size_t)(cur.row0 + rr) * a.H + col));
                }
            }
        }
        wait_vmcnt<0>();
        if (!has_next) break;
        if (more_here) {
            ++u;
        } else {
            item = next_item;
            cur = nxt;
            u = 0;
        }
    }
}

template <class C>
moe_status run_fused(FusedArgs a, int R, hipStream_t s)
{
    auto kern = fused_ffn_kernel<C>;
    static const int occ = [] {  // once per kernel (thread-safe static initialisation)
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_ffn_kernel<C>, C::NT, 0) != hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    const int n2 = (a.H + C::BN - 1) / C::BN;
    // Automatic: one workgroup per row tile.  Every further split re-reads the
    // expert's whole w13 to recompute h; measured on the DeepSeek-V3 and
    // Qwen3-shaped layers, time grows about linearly with the split.
    if (a.nsplit <= 0) a.nsplit = 1;
    if (a.nsplit > n2) a.nsplit = n2;
    const long max_items = ((long)R / C::BM + a.G) * a.nsplit;
    long grid = (long)device_cu_count() * occ;
    if (grid > max_items) grid = max_items;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    {
        TimedLaunch tl(MOE_KID_FFN_FUSED, s);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, a);
    }
    return launch_status("fused_ffn_kernel");
}

// Shapes, measured on MI355X.  16-row tiles: h of 16 rows x 2048 channels is
// 64 KB in bf16, which with the ring fills the LDS; 4 waves split the columns.
//   bf16:         128-column sub-tiles, 4-deep ring (256 columns with a 2-deep
//                 ring: DeepSeek-V3 decode +29%; a 5-deep ring: no gain);
//   fp8 weights:  256-column sub-tiles, 3-deep ring (128 columns, 6-deep:
//                 DeepSeek-V3 decode 5.4 -> 3.4 ms, Qwen3-shaped 5.8 -> 3.4 ms);
//   fp8 x fp8:    256-column sub-tiles (one 128-channel block of h each).  h
//                 codes take half the bytes, so groups averaging 64 rows or
//                 more get 32-row tiles (each expert's weights stream through
//                 the CUs half as often; 2-deep ring: DeepSeek-V3 prefill 17.8
//                 -> 13.7 ms), smaller ones 16-row tiles with a 3-deep ring
//                 (32-row tiles: DeepSeek-V3 decode 2.6 -> 3.5 ms).
using FusedBf16 = FusedCfg<16, 128, 4, 4, false, false, 2 * MOE_FUSED_MAX_I>;
using FusedW8 = FusedCfg<16, 256, 4, 3, true, false, 2 * MOE_FUSED_MAX_I>;
using FusedA8 = FusedCfg<16, 256, 4, 3, true, true, MOE_FUSED_MAX_I>;
using FusedA8Tall = FusedCfg<32, 256, 4, 2, true, true, MOE_FUSED_MAX_I>;
constexpr int kTallRows = 64;  // average rows per group from which fp8 x fp8 takes 32-row tiles

}  // namespace

moe_status launch_ffn_fused(const void* x, const float* x_scale, int act, int T, int H, int I, int k,
                            int E, int n_shared, const int32_t* offsets, const int32_t* permuted_pair,
                            const void* w13, const void* w2, int wdt, const float* w13_scale,
                            const float* w2_scale, int split, void* fc2_out, hipStream_t s)
{
    FusedArgs a{};
    a.x = static_cast<const char*>(x);
    a.xscale = x_scale;
    a.w13 = static_cast<const char*>(w13);
    a.w13s = w13_scale;
    a.w2 = static_cast<const char*>(w2);
    a.w2s = w2_scale;
    a.out = static_cast<char*>(fc2_out);
    a.offsets = offsets;
    a.permuted_pair = permuted_pair;
    a.T = T; a.k = k; a.E = E; a.G = E + n_shared; a.H = H; a.I = I;
    a.nsplit = split;
    const int R = T * k + n_shared * T;
    if (act == MOE_FP8_E4M3)
        return R >= kTallRows * a.G ? run_fused<FusedA8Tall>(a, R, s) : run_fused<FusedA8>(a, R, s);
    if (wdt == MOE_FP8_E4M3) return run_fused<FusedW8>(a, R, s);
    return run_fused<FusedBf16>(a, R, s);
}

}  // namespace moe

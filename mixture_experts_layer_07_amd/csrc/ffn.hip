// moe_expert_ffn: two grouped GEMMs on MFMA.
//
//   FC1 + SwiGLU   h[r, c]   = silu(x_t . W1_g[c]) * (x_t . W3_g[c])   c < I
//   FC2            out[r, n] = h[r] . W2_g[n]                          n < H
//
// for every row r of group g (rows of a group are contiguous after the
// permute; token t = permuted_pair[r] / k for routed groups, r - offsets[g]
// for shared ones).  Weight layout w13 [G, 2I, H] (gate rows then up rows) and
// w2 [G, H, I] as on the vLLM page ("专家权重如何存储"); gated FC1 with 2*I
// outputs as on the TensorRT-LLM page ("权重加载").
//
// Scheduling.  One launch covers every group: the work list is the flattened
// set of (group, N-tile, M-tile) triples ("从 Dense GEMM 到 TP MoE 的演进逻辑",
// section 2.2: tile scheduling over all groups beats one block per group when
// row counts are uneven).  Each workgroup derives the list from the offsets on
// the device (no host read-back), so the launch is graph-capturable.  The grid
// is persistent (sized by CU count and occupancy); workgroups stride through
// the list with an XCD-aware mapping: workgroup b runs on XCD b % 8, and in
// each round XCD x takes one contiguous slice of the list, so the M-tiles that
// share a weight tile run together on the same XCD and share its L2.
//
// Tile engine.  Both operands are K-contiguous (activation rows and weight
// rows), staged through LDS in 128-byte K slices (64 bf16 or 32 fp32 values
// per row) with a 16-byte pad per row (conflict-free 16-byte fragment reads).
// Double-buffered LDS with one barrier per K slice; the next slice's global
// loads are in flight while MFMAs run on the current one.
//   bf16:  v_mfma_f32_16x16x32_bf16; a lane feeds 8 consecutive K values of one
//          row of A and of B.
//   fp32:  v_mfma_f32_16x16x4f32, four per 16-byte fragment (lane group q
//          feeds K = 4q + i to the i-th MFMA, the same for A and B, so the
//          four products cover the 16 K values once).
//   fp8 weights: codes are widened to bf16 while being staged into LDS (exact:
//          every e4m3 value is a bf16 value); the fp32 block scale (one per
//          128x128 block) is constant over each 128-wide K block, so each K
//          block accumulates unscaled into a partial tile which is then added
//          with its scale.
// FC1 keeps the gate and up halves of an output column in the same lane: the
// staged B tile alternates 16 gate rows and the matching 16 up rows, so MFMA
// column blocks 2q and 2q+1 are gate and up of the same 16 outputs and the
// SwiGLU epilogue needs no data exchange.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace moe {
namespace {

enum Mode { FC1 = 0, FC2 = 1 };

struct FfnArgs {
    const char* a_src;         // FC1: x [T, H];  FC2: h [R, I]
    const char* w;             // FC1: w13 [G, 2I, H];  FC2: w2 [G, H, I]
    const float* wscale;       // fp8 block scales or null
    char* out;                 // FC1: h [R, I];  FC2: fc2_out [R, H]
    const int32_t* offsets;    // [G + 1]
    const int32_t* permuted_pair;
    int T, k, E, G, I;
    int N;                     // GEMM output columns (FC1: 2I, FC2: H)
    int K;                     // reduction length (FC1: H, FC2: I)
    int out_ld;                // FC1: I, FC2: H
};

constexpr int kRowBytes = 128;                 // K slice per row, bytes
constexpr int kLdsStride = kRowBytes + 16;     // padded LDS row
constexpr int kMaxGroups = MOE_MAX_EXPERTS + 64;

template <class AT, class WT, int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * 64;
    static constexpr bool F32 = sizeof(AT) == 4;           // fp32 compute
    static constexpr bool FP8 = sizeof(WT) == 1;
    static constexpr int ESZ = F32 ? 4 : 2;                 // LDS element size
    static constexpr int BK = kRowBytes / ESZ;              // K per slice
    static constexpr int WTM = BM / WM, WTN = BN / WN;      // wave tile
    static constexpr int MI = WTM / 16, NI = WTN / 16;      // MFMA blocks
    static constexpr int A_CH = BM * (kRowBytes / 16) / NT; // 16-B A chunks / thread
    static constexpr int B_GCH = FP8 ? 4 : 8;               // global 16-B chunks per B row
    static constexpr int B_CH = BN * B_GCH / NT;            // B chunks / thread
    static constexpr int LDS_A = BM * kLdsStride;
    static constexpr int LDS_B = BN * kLdsStride;
    static_assert(A_CH >= 1 && BM * 8 % NT == 0, "A tile too small for the block");
    static_assert(B_CH >= 1 && BN * B_GCH % NT == 0, "B tile too small for the block");
    static_assert(WTM % 16 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(!FP8 || BK * 2 == 128 || BK == 128, "fp8 scale blocks");
};

__device__ __forceinline__ f32x4_t mfma_frag(u32x4_t a, u32x4_t b, f32x4_t c, bf16_t)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_frag(u32x4_t a, u32x4_t b, f32x4_t c, float)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
}

// Two OCP e4m3fn codes (low or high half of a 32-bit word) -> packed bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
    return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t* p, float v) { *p = f32_to_bf16(v); }


// Global -> registers: the A and B chunks of K slice kt.
template <class C, class WT>
__device__ __forceinline__ void gload(u32x4_t (&ra)[C::A_CH], u32x4_t (&rb)[C::B_CH],
                                      const char* const (&a_ptr)[C::A_CH],
                                      const bool (&a_ok)[C::A_CH],
                                      const char* const (&b_ptr)[C::B_CH], int kt)
{
    const size_t ka = (size_t)kt * kRowBytes;            // A bytes
    const size_t kb = (size_t)kt * C::BK * sizeof(WT);   // W bytes
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i)
        ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4_t*>(a_ptr[i] + ka) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(b_ptr[i] + kb);
}

// Registers -> LDS buffer `buf` (fp8 weights widened to bf16 on the way).
template <class C>
__device__ __forceinline__ void lstore(char* lds, const u32x4_t (&ra)[C::A_CH],
                                       const u32x4_t (&rb)[C::B_CH], int tid, int buf)
{
    char* la = lds + buf * (C::LDS_A + C::LDS_B);
    char* lb = la + C::LDS_A;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
        const int c = tid + i * C::NT;
        *reinterpret_cast<u32x4_t*>(la + (c >> 3) * kLdsStride + (c & 7) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
        const int c = tid + i * C::NT;
        const int j = c / C::B_GCH, q = c % C::B_GCH;
        if (C::FP8) {
            u32x4_t lo4, hi4;
            lo4.x = fp8x2_to_bf16x2<false>(rb[i].x); lo4.y = fp8x2_to_bf16x2<true>(rb[i].x);
            lo4.z = fp8x2_to_bf16x2<false>(rb[i].y); lo4.w = fp8x2_to_bf16x2<true>(rb[i].y);
            hi4.x = fp8x2_to_bf16x2<false>(rb[i].z); hi4.y = fp8x2_to_bf16x2<true>(rb[i].z);
            hi4.z = fp8x2_to_bf16x2<false>(rb[i].w); hi4.w = fp8x2_to_bf16x2<true>(rb[i].w);
            *reinterpret_cast<u32x4_t*>(lb + j * kLdsStride + q * 32) = lo4;
            *reinterpret_cast<u32x4_t*>(lb + j * kLdsStride + q * 32 + 16) = hi4;
        } else {
            *reinterpret_cast<u32x4_t*>(lb + j * kLdsStride + q * 16) = rb[i];
        }
    }
}

template <class AT, class WT, int MODE, class C>
__global__ __launch_bounds__(C::NT) void grouped_gemm_kernel(FfnArgs a)
{
    using CT = typename std::conditional<C::F32, float, bf16_t>::type;  // MFMA input type
    __shared__ __attribute__((aligned(16))) char lds[2 * (C::LDS_A + C::LDS_B)];
    __shared__ int s_off[kMaxGroups + 1];
    __shared__ int s_tile0[kMaxGroups + 1];  // first flat tile of each group

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int G = a.G;
    const int NTILES_N = (MODE == FC1) ? a.N / C::BN : a.N / C::BN;

    // ---- flattened tile list: group g owns tiles [s_tile0[g], s_tile0[g+1])
    for (int g = tid; g <= G; g += C::NT) s_off[g] = a.offsets[g];
    __syncthreads();
    if (wave == 0) {
        // per lane, a contiguous run of groups; wave-wide exclusive scan
        const int per = (G + 63) / 64;
        const int g0 = lane * per, g1 = min(G, g0 + per);
        int sum = 0;
        for (int g = g0; g < g1; ++g) {
            const int n = max(0, s_off[g + 1] - s_off[g]);
            sum += (n + C::BM - 1) / C::BM * NTILES_N;
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        int run = incl - sum;
        for (int g = g0; g < g1; ++g) {
            s_tile0[g] = run;
            const int n = max(0, s_off[g + 1] - s_off[g]);
            run += (n + C::BM - 1) / C::BM * NTILES_N;
        }
        if (lane == 63) s_tile0[G] = incl;
    }
    __syncthreads();
    const int total = s_tile0[G];

    const int nb = gridDim.x;
    const bool xcd_map = (nb % 8) == 0;
    const int slot = xcd_map ? (blockIdx.x >> 3) + (blockIdx.x & 7) * (nb >> 3) : blockIdx.x;

    const int nk = a.K / C::BK;
    const size_t a_ld = (size_t)((MODE == FC1) ? a.K : a.K) * sizeof(AT);  // A row bytes
    const size_t w_ld = (size_t)a.K * sizeof(WT);                          // W row bytes

    for (int tile = slot; tile < total; tile += nb) {
        // ---- decode tile -> (g, nt, mt)
        int lo = 0, hi = G - 1;
        while (lo < hi) {  // last g with s_tile0[g] <= tile
            const int mid = (lo + hi + 1) >> 1;
            if (s_tile0[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int g = lo;
        const int row0 = s_off[g];
        const int nrows = s_off[g + 1] - row0;
        const int mtiles = (nrows + C::BM - 1) / C::BM;
        const int local = tile - s_tile0[g];
        const int nt = local / mtiles;
        const int mt = local - nt * mtiles;
        const int m0 = mt * C::BM;

        // ---- per-thread global source rows
        const char* a_ptr[C::A_CH];
        bool a_ok[C::A_CH];
#pragma unroll
        for (int i = 0; i < C::A_CH; ++i) {
            const int c = tid + i * C::NT;
            const int r = c >> 3;
            const int rr = m0 + r;
            a_ok[i] = rr < nrows;
            long src;
            if (MODE == FC1) {
                int tok = 0;
                if (a_ok[i]) {
                    tok = (g < a.E) ? a.permuted_pair[row0 + rr] / a.k : rr;
                    tok = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
                }
                src = tok;
            } else {
                src = a_ok[i] ? row0 + rr : 0;
            }
            a_ptr[i] = a.a_src + (size_t)src * a_ld + (size_t)(c & 7) * 16;
        }
        const char* b_ptr[C::B_CH];
#pragma unroll
        for (int i = 0; i < C::B_CH; ++i) {
            const int c = tid + i * C::NT;
            const int j = c / C::B_GCH;  // B tile row
            int wrow;
            if (MODE == FC1) {
                const int blk = j >> 4, pair = blk >> 1;
                const int col = nt * (C::BN / 2) + pair * 16 + (j & 15);
                wrow = (blk & 1) ? a.I + col : col;
            } else {
                wrow = nt * C::BN + j;
            }
            b_ptr[i] = a.w + ((size_t)g * a.N + wrow) * w_ld + (size_t)(c % C::B_GCH) * 16;
        }

        // ---- K loop
        u32x4_t ra[C::A_CH], rb[C::B_CH];
        f32x4_t acc[C::MI][C::NI];
        f32x4_t part[C::FP8 ? C::MI : 1][C::FP8 ? C::NI : 1];
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (C::FP8) {
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) part[C::FP8 ? mi : 0][C::FP8 ? ni : 0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

        gload<C, WT>(ra, rb, a_ptr, a_ok, b_ptr, 0);
        lstore<C>(lds, ra, rb, tid, 0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) gload<C, WT>(ra, rb, a_ptr, a_ok, b_ptr, kt + 1);
            const char* la = lds + buf * (C::LDS_A + C::LDS_B);
            const char* lb = la + C::LDS_A;
#pragma unroll
            for (int ks = 0; ks < kRowBytes / 64; ++ks) {
                u32x4_t fa[C::MI], fb[C::NI];
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
                    fa[mi] = *reinterpret_cast<const u32x4_t*>(
                        la + (wm * C::WTM + mi * 16 + (lane & 15)) * kLdsStride + ks * 64 + (lane >> 4) * 16);
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
                    fb[ni] = *reinterpret_cast<const u32x4_t*>(
                        lb + (wn * C::WTN + ni * 16 + (lane & 15)) * kLdsStride + ks * 64 + (lane >> 4) * 16);
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni) {
                        if (C::FP8)
                            part[C::FP8 ? mi : 0][C::FP8 ? ni : 0] =
                                mfma_frag(fa[mi], fb[ni], part[C::FP8 ? mi : 0][C::FP8 ? ni : 0], CT());
                        else
                            acc[mi][ni] = mfma_frag(fa[mi], fb[ni], acc[mi][ni], CT());
                    }
            }
            if (C::FP8 && ((kt + 1) * C::BK) % 128 == 0) {
                // end of a 128-wide K block: acc += scale * partial
                const int kb = (kt * C::BK) / 128;
                const int sk = a.K / 128;
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    const int j = wn * C::WTN + ni * 16;  // first staged B row of this block
                    int wrow;
                    if (MODE == FC1) {
                        const int blk = j >> 4, pair = blk >> 1;
                        const int col = nt * (C::BN / 2) + pair * 16;
                        wrow = (blk & 1) ? a.I + col : col;
                    } else {
                        wrow = nt * C::BN + j;
                    }
                    const float s = a.wscale[((size_t)g * (a.N / 128) + wrow / 128) * sk + kb];
#pragma unroll
                    for (int mi = 0; mi < C::MI; ++mi) {
                        acc[mi][ni] += s * part[C::FP8 ? mi : 0][C::FP8 ? ni : 0];
                        part[C::FP8 ? mi : 0][C::FP8 ? ni : 0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
                }
            }
            if (kt + 1 < nk) lstore<C>(lds, ra, rb, tid, buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue
        AT* out = reinterpret_cast<AT*>(a.out);
        if (MODE == FC1) {
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int q = 0; q < C::NI / 2; ++q) {
                    const int pair = (wn * C::WTN) / 32 + q;
                    const int col = nt * (C::BN / 2) + pair * 16 + (lane & 15);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = m0 + wm * C::WTM + mi * 16 + (lane >> 4) * 4 + i;
                        if (rr < nrows) {
                            const float gt = acc[mi][2 * q][i];
                            const float up = acc[mi][2 * q + 1][i];
                            const float hv = gt / (1.0f + expf(-gt)) * up;
                            store_out(out + (size_t)(row0 + rr) * a.out_ld + col, hv);
                        }
                    }
                }
        } else {
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    const int col = nt * C::BN + wn * C::WTN + ni * 16 + (lane & 15);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = m0 + wm * C::WTM + mi * 16 + (lane >> 4) * 4 + i;
                        if (rr < nrows) store_out(out + (size_t)(row0 + rr) * a.out_ld + col, acc[mi][ni][i]);
                    }
                }
        }
    }
}

struct DevInfo {
    int cus = 0;
};

template <class AT, class WT, int MODE, class C>
moe_status run_gemm(const FfnArgs& args, int rows_upper, int ntiles_n, hipStream_t s, int kid)
{
    auto kern = grouped_gemm_kernel<AT, WT, MODE, C>;
    static int occ = -1;
    if (occ < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, C::NT, 0) != hipSuccess || n < 1) n = 1;
        occ = n;
    }
    const long max_tiles = (long)((rows_upper + C::BM - 1) / C::BM + args.G) * ntiles_n;
    long grid = (long)device_cu_count() * occ;
    if (grid > max_tiles) grid = max_tiles;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    {
        TimedLaunch tl(kid, s);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, args);
    }
    return launch_status(MODE == FC1 ? "fc1 grouped_gemm_kernel" : "fc2 grouped_gemm_kernel");
}

template <class AT, class WT>
moe_status run_ffn(const FfnArgs& fc1, const FfnArgs& fc2, int R, int G, hipStream_t s)
{
    // Tile shape from the mean rows per group: skinny groups (decode-like)
    // stream weights with a 32-row tile; larger groups use 128x128.
    const bool skinny = R <= 48 * G;
    moe_status st;
    if (skinny) {
        using C = Cfg<AT, WT, 32, 128, 1, 4>;
        st = run_gemm<AT, WT, FC1, C>(fc1, R, fc1.N / C::BN, s, MOE_KID_FC1);
        if (st != MOE_OK) return st;
        return run_gemm<AT, WT, FC2, C>(fc2, R, fc2.N / C::BN, s, MOE_KID_FC2);
    } else {
        using C = Cfg<AT, WT, 128, 128, 2, 2>;
        st = run_gemm<AT, WT, FC1, C>(fc1, R, fc1.N / C::BN, s, MOE_KID_FC1);
        if (st != MOE_OK) return st;
        return run_gemm<AT, WT, FC2, C>(fc2, R, fc2.N / C::BN, s, MOE_KID_FC2);
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t ffn_scratch_bytes(int T, int k, int n_shared, int I, int act)
{
    const size_t R = (size_t)T * k + (size_t)n_shared * T;
    return align256(R * (size_t)I * (act == MOE_F32 ? 4 : 2));
}

moe_status launch_ffn(const void* x, int act, int T, int H, int I, int k, int E, int n_shared,
                      const int32_t* offsets, const int32_t* permuted_pair, const void* w13,
                      const void* w2, int wdt, const float* w13_scale, const float* w2_scale,
                      void* fc2_out, void* ws, hipStream_t s)
{
    const int G = E + n_shared;
    const int R = T * k + n_shared * T;
    FfnArgs f1{};
    f1.a_src = static_cast<const char*>(x);
    f1.w = static_cast<const char*>(w13);
    f1.wscale = w13_scale;
    f1.out = static_cast<char*>(ws);
    f1.offsets = offsets;
    f1.permuted_pair = permuted_pair;
    f1.T = T; f1.k = k; f1.E = E; f1.G = G; f1.I = I;
    f1.N = 2 * I; f1.K = H; f1.out_ld = I;
    FfnArgs f2 = f1;
    f2.a_src = static_cast<const char*>(ws);
    f2.w = static_cast<const char*>(w2);
    f2.wscale = w2_scale;
    f2.out = static_cast<char*>(fc2_out);
    f2.N = H; f2.K = I; f2.out_ld = H;
    if (act == MOE_F32) return run_ffn<float, float>(f1, f2, R, G, s);
    if (wdt == MOE_FP8_E4M3) return run_ffn<bf16_t, fp8_t>(f1, f2, R, G, s);
    return run_ffn<bf16_t, bf16_t>(f1, f2, R, G, s);
}

}  // namespace moe

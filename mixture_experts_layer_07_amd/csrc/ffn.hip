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
// Scheduling.  Work is a flattened list of (group, N-tile, M-tile) triples
// ("从 Dense GEMM 到 TP MoE 的演进逻辑", section 2.2: tile scheduling over all
// groups beats one block per group when row counts are uneven).  Groups are
// split by row count into three classes (skinny, mid, big), and each GEMM is
// issued as one launch per class, back to back on the caller's stream, each
// with the tile shape that suits its class (run_classes_dma below); a launch's
// list holds the tiles of its class's groups only.  Each workgroup derives its
// launch's list from the offsets on the device (no host read-back), so the
// launches are graph-capturable.  The grid is persistent (sized by CU count
// and occupancy); workgroups stride through the list with an XCD-aware
// mapping: workgroup b runs on XCD b % 8, and in each round XCD x takes one
// contiguous slice of the list, so the M-tiles that share a weight tile run
// together on the same XCD and share its L2.
//
// Two tile engines.  Both operands are K-contiguous (activation rows and
// weight rows), staged through LDS in 128-byte K slices whose 16-byte chunks
// are XOR-swizzled by row (conflict-free).
//   Register-staged engine (fp32 layers): global -> VGPR -> LDS, double
//          buffered, one barrier per slice; v_mfma_f32_16x16x4f32, four per
//          16-byte fragment (lane group q feeds K = 4q + i to the i-th MFMA,
//          the same for A and B, so the four products cover the 16 K values
//          once).
//   Direct-to-LDS engine (bf16 activations with bf16 or fp8 weights, or
//          fp8 activations with fp8 weights): described at DmaCfg below;
//          v_mfma_f32_16x16x32_bf16, a lane feeding 8 consecutive K values
//          of one row of A and of B, or v_mfma_f32_16x16x128_f8f6f4 with 32.
// FC1 keeps the gate and up halves of an output column in the same lane: the
// staged B tile alternates 16 gate rows and the matching 16 up rows, so MFMA
// column blocks 2q and 2q+1 are gate and up of the same 16 outputs and the
// SwiGLU epilogue needs no data exchange.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "dma.h"

namespace moe {
namespace {

enum Mode { FC1 = 0, FC2 = 1 };

struct FfnArgs {
    const char* a_src;         // FC1: x [T, H];  FC2: h [R, I]
    const char* w;             // FC1: w13 [G, 2I, H];  FC2: w2 [G, H, I]
    const float* wscale;       // fp8 block scales or null
    const float* ascale;       // fp8 activations: FC1 x scales [T, H/128], FC2 h scales [R, I/128]
    float* out_scale;          // fp8 activations, FC1: h scales [R, I/128] out
    char* out;                 // FC1: h [R, I];  FC2: fc2_out [R, H]
    const int32_t* offsets;    // [G + 1]
    const int32_t* permuted_pair;
    int T, k, E, G, I;
    int N;                     // GEMM output columns (FC1: 2I, FC2: H)
    int K;                     // reduction length (FC1: H, FC2: I)
    int out_ld;                // FC1: I, FC2: H
    int lo_rows, hi_rows;      // this launch serves groups with lo <= rows < hi
    // Remainder hand-off between row classes: a launch whose own group ends in
    // a partial tile of at most give_max rows leaves those rows out; the launch
    // with take_max > 0 serves them for groups of [take_lo, take_hi) (whose
    // tile height was take_bm).  0 = no hand-off.
    int give_max;
    int take_lo, take_hi, take_bm, take_max;
};

// Rows [beg, end) of a group of n rows that a launch with tile height bm
// serves (see FfnArgs); beg == end when it serves none.
struct RowWindow {
    int beg, end;
};
__device__ __forceinline__ RowWindow row_window(const FfnArgs& a, int n, int bm)
{
    if (n >= a.lo_rows && n < a.hi_rows && n > 0) {
        const int r = n % bm;
        return {0, (a.give_max > 0 && n >= bm && r >= 1 && r <= a.give_max) ? n - r : n};
    }
    if (a.take_max > 0 && n >= a.take_lo && n < a.take_hi && n >= a.take_bm) {
        const int r = n % a.take_bm;
        if (r >= 1 && r <= a.take_max) return {n - r, n};
    }
    return {0, 0};
}

constexpr int kRowBytes = 128;                 // K slice per row, bytes
constexpr int kLdsStride = kRowBytes;          // LDS row (no pad: XOR-swizzled chunks)

// LDS byte offset of 16-byte chunk `kc` (0..7) of staged row `row`.  The chunk
// index is XORed with row % 8: measured on gfx950, this makes both the
// fragment reads (16 rows x 4 chunks per ds_read_b128) and the staging writes
// (8 lanes per row) free of bank conflicts, where a padded 144-byte row is not.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * kLdsStride + ((kc ^ (row & 7)) << 4); }

template <class AT, class WT, int BM_, int BN_, int WM_, int WN_, int GM_ = 1>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, GM = GM_;
    static constexpr int NT = WM * WN * 64;
    static constexpr bool F32 = sizeof(AT) == 4;           // fp32 compute
    static constexpr int ESZ = F32 ? 4 : 2;                 // LDS element size
    static constexpr int BK = kRowBytes / ESZ;              // K per slice
    static constexpr int WTM = BM / WM, WTN = BN / WN;      // wave tile
    static constexpr int MI = WTM / 16, NI = WTN / 16;      // MFMA blocks
    static constexpr int A_CH = BM * (kRowBytes / 16) / NT; // 16-B A chunks / thread
    static constexpr int B_GCH = 8;                         // global 16-B chunks per B row
    static constexpr int B_CH = BN * B_GCH / NT;            // B chunks / thread
    static constexpr int LDS_A = BM * kLdsStride;
    static constexpr int LDS_B = BN * kLdsStride;
    static_assert(A_CH >= 1 && BM * 8 % NT == 0, "A tile too small for the block");
    static_assert(B_CH >= 1 && BN * B_GCH % NT == 0, "B tile too small for the block");
    static_assert(WTM % 16 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(sizeof(AT) == sizeof(WT) && sizeof(WT) >= 2, "fp32 or bf16 operands");
};

// fp32 form of mfma_frag: four 16x16x4 MFMAs over the 16-byte fragments.
__device__ __forceinline__ f32x4_t mfma_frag(u32x4_t a, u32x4_t b, f32x4_t c, float)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// Four consecutive bf16 outputs (8 bytes, 8-byte aligned)
__device__ __forceinline__ void store4_bf16(bf16_t* p, const float (&v)[4])
{
    const unsigned lo = pack_bf16x2(v[0], v[1]);
    const unsigned hi = pack_bf16x2(v[2], v[3]);
    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
    *(__attribute__((address_space(1))) u32x2_t*)(p) = u32x2_t{lo, hi};
}


// 16-byte load through the global address space.  The tile pointers live in
// a by-value struct and loop-carried registers, where the compiler cannot infer
// the address space and would emit flat loads, which also count against the
// LDS wait counter and so serialise the global latency with LDS traffic.
__device__ __forceinline__ u32x4_t ldg16(const char* p)
{
    return *(const __attribute__((address_space(1))) u32x4_t*)(p);
}

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
        ra[i] = a_ok[i] ? ldg16(a_ptr[i] + ka) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) rb[i] = ldg16(b_ptr[i] + kb);
}

// Registers -> LDS buffer `buf`.
template <class C>
__device__ __forceinline__ void lstore(char* lds, const u32x4_t (&ra)[C::A_CH],
                                       const u32x4_t (&rb)[C::B_CH], int tid, int buf)
{
    char* la = lds + buf * (C::LDS_A + C::LDS_B);
    char* lb = la + C::LDS_A;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
        const int c = tid + i * C::NT;
        *reinterpret_cast<u32x4_t*>(la + lds_off(c >> 3, c & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
        const int c = tid + i * C::NT;
        const int j = c / C::B_GCH, q = c % C::B_GCH;
        *reinterpret_cast<u32x4_t*>(lb + lds_off(j, q)) = rb[i];
    }
}

// Tile of the flattened work list, decoded.
// nrows: end of the rows this launch serves in group g (rows >= nrows of a
// tile are padding); m0: first row of the tile within the group.
struct TileInfo {
    int g, row0, nrows, m0, nt;
};

template <class C>
__device__ __forceinline__ TileInfo decode_tile(const FfnArgs& a, int tile, const int* s_off,
                                                const int* s_tile0, int G, int ntiles_n)
{
    // every value here is block-uniform; readfirstlane keeps them in SGPRs
    int lo = 0, hi = G - 1;
    while (lo < hi) {  // last g with s_tile0[g] <= tile
        const int mid = (lo + hi + 1) >> 1;
        if (__builtin_amdgcn_readfirstlane(s_tile0[mid]) <= tile) lo = mid; else hi = mid - 1;
    }
    TileInfo ti;
    ti.g = lo;
    ti.row0 = __builtin_amdgcn_readfirstlane(s_off[lo]);
    const RowWindow win = row_window(a, __builtin_amdgcn_readfirstlane(s_off[lo + 1]) - ti.row0, C::BM);
    ti.nrows = win.end;
    const int mtiles = (win.end - win.beg + C::BM - 1) / C::BM;
    // group-M order: runs of GM M-tiles share one N-tile, so a contiguous slice
    // of the list reuses both operands (A across N-tiles, B across M-tiles)
    const int local = tile - __builtin_amdgcn_readfirstlane(s_tile0[lo]);
    const int band = local / (C::GM * ntiles_n);
    const int first_m = band * C::GM;
    const int gm = min(mtiles - first_m, C::GM);
    const int r = local - band * C::GM * ntiles_n;
    ti.m0 = win.beg + (first_m + r % gm) * C::BM;
    ti.nt = r / gm;
    return ti;
}

// Per-thread global source pointers of a tile's A rows and B (weight) rows.
template <class AT, class WT, int MODE, class C>
__device__ __forceinline__ void tile_pointers(const FfnArgs& a, const TileInfo& ti, int tid,
                                              const char* (&a_ptr)[C::A_CH], bool (&a_ok)[C::A_CH],
                                              const char* (&b_ptr)[C::B_CH])
{
    const size_t a_ld = (size_t)a.K * sizeof(AT);
    const size_t w_ld = (size_t)a.K * sizeof(WT);
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
        const int c = tid + i * C::NT;
        const int rr = ti.m0 + (c >> 3);
        a_ok[i] = rr < ti.nrows;
        long src = 0;
        if (a_ok[i]) {
            if (MODE == FC1) {
                int tok = (ti.g < a.E) ? a.permuted_pair[ti.row0 + rr] / a.k : rr;
                src = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            } else {
                src = ti.row0 + rr;
            }
        }
        a_ptr[i] = a.a_src + (size_t)src * a_ld + (size_t)(c & 7) * 16;
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
        const int c = tid + i * C::NT;
        const int j = c / C::B_GCH;  // staged B row
        int wrow;
        if (MODE == FC1) {
            const int blk = j >> 4, pair = blk >> 1;
            const int col = ti.nt * (C::BN / 2) + pair * 16 + (j & 15);
            wrow = (blk & 1) ? a.I + col : col;
        } else {
            wrow = min(ti.nt * C::BN + j, a.N - 1);  // partial last N-tile: rows past N unused
        }
        b_ptr[i] = a.w + ((size_t)ti.g * a.N + wrow) * w_ld + (size_t)(c % C::B_GCH) * 16;
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
    // FC2's N (= H) is a multiple of 128 only: the last N-tile may be partial
    const int ntiles_n = (a.N + C::BN - 1) / C::BN;

    // ---- flattened tile list of the groups in this launch's row class
    //      [a.lo_rows, a.hi_rows): group g owns tiles [s_tile0[g], s_tile0[g+1])
    for (int g = tid; g <= G; g += C::NT) s_off[g] = a.offsets[g];
    __syncthreads();
    if (wave == 0) {
        const int per = (G + 63) / 64;  // a contiguous run of groups per lane
        const int g0 = lane * per, g1 = min(G, g0 + per);
        auto ntiles = [&](int g) {
            const int n = s_off[g + 1] - s_off[g];
            const RowWindow w = row_window(a, n, C::BM);
            return (w.end - w.beg + C::BM - 1) / C::BM * ntiles_n;
        };
        int sum = 0;
        for (int g = g0; g < g1; ++g) sum += ntiles(g);
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        int run = incl - sum;
        for (int g = g0; g < g1; ++g) {
            s_tile0[g] = run;
            run += ntiles(g);
        }
        if (lane == 63) s_tile0[G] = incl;
    }
    __syncthreads();
    const int total = s_tile0[G];

    const int nb = gridDim.x;
    const bool xcd_map = (nb % 8) == 0;
    const int slot = xcd_map ? (blockIdx.x >> 3) + (blockIdx.x & 7) * (nb >> 3) : blockIdx.x;
    int tile = slot;
    if (tile >= total) return;

    const int nk = a.K / C::BK;
    const char* a_ptr[C::A_CH];
    bool a_ok[C::A_CH];
    const char* b_ptr[C::B_CH];
    u32x4_t ra[C::A_CH], rb[C::B_CH];

    TileInfo cur = decode_tile<C>(a, tile, s_off, s_tile0, G, ntiles_n);
    tile_pointers<AT, WT, MODE, C>(a, cur, tid, a_ptr, a_ok, b_ptr);
    gload<C, WT>(ra, rb, a_ptr, a_ok, b_ptr, 0);
    lstore<C>(lds, ra, rb, tid, 0);
    __syncthreads();
    int buf = 0;

    while (true) {
        const int next_tile = tile + nb;
        const bool has_next = next_tile < total;
        TileInfo nxt = cur;

        f32x4_t acc[C::MI][C::NI];
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < C::NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int kt = 0; kt < nk; ++kt) {
            // issue the next slice's loads: this tile's, or the next tile's first
            bool staged = true;
            if (kt + 1 < nk) {
                gload<C, WT>(ra, rb, a_ptr, a_ok, b_ptr, kt + 1);
            } else if (has_next) {
                nxt = decode_tile<C>(a, next_tile, s_off, s_tile0, G, ntiles_n);
                tile_pointers<AT, WT, MODE, C>(a, nxt, tid, a_ptr, a_ok, b_ptr);
                gload<C, WT>(ra, rb, a_ptr, a_ok, b_ptr, 0);
            } else {
                staged = false;
            }
            const char* la = lds + buf * (C::LDS_A + C::LDS_B);
            const char* lb = la + C::LDS_A;
#pragma unroll
            for (int ks = 0; ks < kRowBytes / 64; ++ks) {
                u32x4_t fa[C::MI], fb[C::NI];
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
                    fa[mi] = *reinterpret_cast<const u32x4_t*>(
                        la + lds_off(wm * C::WTM + mi * 16 + (lane & 15), ks * 4 + (lane >> 4)));
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni)
                    fb[ni] = *reinterpret_cast<const u32x4_t*>(
                        lb + lds_off(wn * C::WTN + ni * 16 + (lane & 15), ks * 4 + (lane >> 4)));
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni) acc[mi][ni] = mfma_frag(fa[mi], fb[ni], acc[mi][ni], CT());
            }
            if (staged) lstore<C>(lds, ra, rb, tid, buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }

        // ---- epilogue (registers -> global; the next tile's first slice is in LDS)
        AT* out = reinterpret_cast<AT*>(a.out);
        if (MODE == FC1) {
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int q = 0; q < C::NI / 2; ++q) {
                    const int pair = (wn * C::WTN) / 32 + q;
                    const int col = cur.nt * (C::BN / 2) + pair * 16 + (lane & 15);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = cur.m0 + wm * C::WTM + mi * 16 + (lane >> 4) * 4 + i;
                        if (rr < cur.nrows) {
                            const float gt = acc[mi][2 * q][i];
                            const float up = acc[mi][2 * q + 1][i];
                            // silu(g) * u; v_rcp_f32 (1 ulp) instead of an IEEE divide
                            const float hv = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * up;
                            store_out(out + (size_t)(cur.row0 + rr) * a.out_ld + col, hv);
                        }
                    }
                }
        } else {
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    const int col = cur.nt * C::BN + wn * C::WTN + ni * 16 + (lane & 15);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = cur.m0 + wm * C::WTM + mi * 16 + (lane >> 4) * 4 + i;
                        if (rr < cur.nrows && col < a.N)
                            store_out(out + (size_t)(cur.row0 + rr) * a.out_ld + col, acc[mi][ni][i]);
                    }
                }
        }
        if (!has_next) break;
        tile = next_tile;
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// Tile engine with direct global->LDS loads (bf16 activations with bf16 or
// fp8 weights; fp8 activations with fp8 weights).
//
// Each stage is one K slice: BM activation rows of 128 bytes (64 bf16 or 128
// fp8 values) and BN weight rows of 128 bytes, or 64 bytes for fp8 weights
// under bf16 activations, written straight into LDS by
// global_load_lds_dwordx4: one instruction moves 1 KB, lane l landing at byte
// 16*l, i.e. 8 rows of 128 bytes or 16 of 64, every lane request a full line
// or half line.  Sources are a scalar base (activations, the tile's expert
// weights, activation scales) plus a 32-bit per-lane offset.  A ring of S
// stages keeps S-1 slices in flight without holding anything in VGPRs; one
// LDS-only barrier per slice.  The next tile's token indices are fetched when
// a tile starts and its first slices are issued before the current tile's
// epilogue, so a tile change exposes only the epilogue.
//
// fp8 weights (W8): a lane reads its 8 fp8 values of a fragment from LDS and
// widens them to bf16 (exact: every e4m3 value is a bf16 value); the MFMA
// sums of one 128-wide K block go into a partial tile that is added to the
// accumulator times the block's fp32 scale (exact in the scale), so the only
// rounding besides fp32 accumulation is the one of the output.
//
// fp8 activations (A8, with fp8 weights): a stage is one 128-wide K block,
// 128-byte rows of fp8 codes for both operands, multiplied on
// v_mfma_f32_16x16x128_f8f6f4 (exact products; the instruction's own sum of
// 128 products is not exactly rounded fp32, ~13 bits measured, hence one
// MFMA per block and fp32 accumulation across blocks).  Each wave also stages
// the 1x128 activation scales of its own WTM rows for that block (one
// 4-byte-per-lane transfer into a private 256-byte slot), and adds each
// block's MFMA result to the accumulator times (row scale x weight-block
// scale), software-pipelined one MFMA behind.  FC1's epilogue quantises h per
// row and 128 intermediate channels (one 256-column tile holds exactly one
// such block of every row).
template <int BM_, int BN_, int WM_, int WN_, int GM_, int S_, bool W8_ = false, bool A8_ = false>
struct DmaCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, GM = GM_, S = S_;
    static constexpr bool A8 = A8_;
    static constexpr bool W8 = W8_ || A8_;                 // fp8 weights
    static constexpr bool WNARROW = W8 && !A8;             // fp8 weights widened to bf16
    static constexpr int NT = WM * WN * 64;
    static constexpr int NW = WM * WN;
    static constexpr int BK = A8 ? 128 : 64;               // K per stage
    static constexpr int KSTEPS = A8 ? 1 : BK / 32;        // MFMA K-steps per stage
    static constexpr int BROWB = WNARROW ? 64 : 128;       // weight bytes per staged row
    static constexpr int A_OPS = BM / 8;                   // 1 KB DMA ops per stage, activations
    static constexpr int B_OPS = BN * BROWB / 1024;        // ... and weights
    static constexpr int A_BYTES = BM * 128;
    static constexpr int B_BYTES = BN * BROWB;
    static constexpr int SA_BYTES = A8 ? NW * 256 : 0;     // per-wave activation-scale slots
    static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;  // bytes per stage
    static constexpr int NINS = A_OPS + B_OPS;
    static constexpr int IPW_AB = NINS / NW;               // 1 KB ops per wave per stage
    static constexpr int IPW = IPW_AB + (A8 ? 1 : 0);      // ... plus the scale transfer
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MI = WTM / 16, NI = WTN / 16;
    static constexpr int AMAX_BYTES = A8 ? BM * WN * 4 : 4;  // FC1 epilogue: row maxima per wave column
    static_assert(BM % 8 == 0 && NINS % NW == 0 && IPW_AB >= 1, "DMA ops split evenly over waves");
    static_assert(WTM % 16 == 0 && WTN % 32 == 0, "tile");
    static_assert(!A8 || (WTM <= 64 && BN == 256), "A8: one scale transfer per wave; 128 h columns per tile");
    static_assert(S >= 2 && S <= 8 && S * STAGE + AMAX_BYTES <= 156 * 1024,
                  "ring (LDS also holds the tile tables)");
};


template <int MODE, class C>
__global__ __launch_bounds__(C::NT) void dma_gemm_kernel(FfnArgs a)
{
    __shared__ __attribute__((aligned(1024))) char lds[C::S * C::STAGE];
    __shared__ int s_off[kMaxGroups + 1];
    __shared__ int s_tile0[kMaxGroups + 1];
    __shared__ float s_amax[C::AMAX_BYTES / 4];  // A8 FC1 epilogue: [BM][WN] row maxima

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave values stay in SGPRs
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int G = a.G;
    const int ntiles_n = (a.N + C::BN - 1) / C::BN;

    // ---- flattened tile list of this launch's row class (as in grouped_gemm_kernel)
    for (int g = tid; g <= G; g += C::NT) s_off[g] = a.offsets[g];
    __syncthreads();
    if (wave == 0) {
        const int per = (G + 63) / 64;
        const int g0 = lane * per, g1 = min(G, g0 + per);
        auto ntiles = [&](int g) {
            const int n = s_off[g + 1] - s_off[g];
            const RowWindow w = row_window(a, n, C::BM);
            return (w.end - w.beg + C::BM - 1) / C::BM * ntiles_n;
        };
        int sum = 0;
        for (int g = g0; g < g1; ++g) sum += ntiles(g);
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        int run = incl - sum;
        for (int g = g0; g < g1; ++g) {
            s_tile0[g] = run;
            run += ntiles(g);
        }
        if (lane == 63) s_tile0[G] = incl;
    }
    __syncthreads();
    const int total = s_tile0[G];
    const int nb = gridDim.x;
    const bool xcd_map = (nb % 8) == 0;
    const int slot = xcd_map ? (blockIdx.x >> 3) + (blockIdx.x & 7) * (nb >> 3) : blockIdx.x;
    int tile = slot;
    if (tile >= total) return;

    const int nk = a.K / C::BK;
    const size_t a_ld = (size_t)a.K * (C::A8 ? 1 : 2), w_ld = (size_t)a.K * (C::W8 ? 1 : 2);
    const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)lds;

    // Op o = q*NW + wave of a stage (wave-uniform, q < IPW_AB) stages
    // activation rows 8o .. 8o+7 when o < A_OPS, else weight rows: 8 rows of
    // 128 bytes or 16 narrow fp8 rows of 64 bytes from row (o - A_OPS) *
    // rows-per-op.  Lane l writes the op's LDS bytes [16l, 16l+16): row l / 8
    // (l / 4 for narrow rows) of the op, physical chunk l % 8 (l % 4), which
    // holds logical chunk physical ^ swizzle(row).  With fp8 activations op
    // q = IPW_AB of every wave stages the activation scales of the wave's own
    // rows: lane l fetches the scale of row wm*WTM + l % WTM.
    auto op_is_s = [&](int q) { return C::A8 && q == C::IPW_AB; };
    auto op_is_a = [&](int q) { return q < C::IPW_AB && q * C::NW + wave < C::A_OPS; };
    auto op_row = [&](int q) {  // A row, or B row, of this lane in op q < IPW_AB
        const int o = q * C::NW + wave;
        if (o < C::A_OPS) return o * 8 + (lane >> 3);
        return C::WNARROW ? (o - C::A_OPS) * 16 + (lane >> 2) : (o - C::A_OPS) * 8 + (lane >> 3);
    };
    auto op_chunk = [&](int q, int row) {  // logical 16-byte chunk this lane fetches
        if (op_is_a(q) || !C::WNARROW) return (lane & 7) ^ (row & 7);
        return (lane & 3) ^ ((row >> 2) & 3);
    };
    const int s_row = wm * C::WTM + lane % C::WTM;  // scale op: this lane's tile row

    // For FC1 A rows the token comes from permuted_pair: a_raw() only loads the
    // entry (from an always-valid address) and source() interprets it, so the
    // next tile's loads can be issued early and consumed a whole tile later.
    auto a_raw = [&](const TileInfo& ti, int q) -> int {
        if (MODE == FC2 || !(op_is_a(q) || op_is_s(q))) return 0;
        const int rr = ti.m0 + (op_is_s(q) ? s_row : op_row(q));
        const int i = (ti.g < a.E && rr < ti.nrows) ? ti.row0 + rr : 0;
        // global-space load: a flat load would also count in lgkmcnt and make
        // the LDS-only barriers wait for it
        return *(const __attribute__((address_space(1))) int*)(a.permuted_pair + i);
    };
    // Per-lane byte offset of op q's source from its base: the activations
    // (a_src), this tile's group of weights (wbase) or the activation scales.
    auto source = [&](const TileInfo& ti, int q, int raw) -> uint32_t {
        if (op_is_s(q)) {
            const int rr = ti.m0 + s_row;
            long r;
            if (MODE == FC1) {
                const int tok = (rr >= ti.nrows) ? 0 : (ti.g < a.E ? raw / a.k : rr);
                r = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            } else {
                r = ti.row0 + (rr < ti.nrows ? rr : 0);
            }
            return (uint32_t)(r * (a.K / 128) * 4);
        }
        const int row = op_row(q);
        uint32_t p;
        if (op_is_a(q)) {
            const int rr = ti.m0 + row;
            long r;
            if (MODE == FC1) {
                int tok = (rr >= ti.nrows) ? 0 : (ti.g < a.E ? raw / a.k : rr);  // padding rows: token 0
                r = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            } else {
                r = ti.row0 + (rr < ti.nrows ? rr : 0);
            }
            p = (uint32_t)(r * a_ld);
        } else {
            const int j = row;
            int wrow;
            if (MODE == FC1) {
                const int blk = j >> 4, pair = blk >> 1;
                const int col = ti.nt * (C::BN / 2) + pair * 16 + (j & 15);
                wrow = (blk & 1) ? a.I + col : col;
            } else {
                wrow = min(ti.nt * C::BN + j, a.N - 1);  // partial last N-tile
            }
            p = (uint32_t)(wrow * w_ld);
        }
        return p + op_chunk(q, row) * 16;
    };
    auto group_weights = [&](const TileInfo& ti) { return uniform_ptr(a.w + (size_t)ti.g * a.N * w_ld); };
    const char* abase = uniform_ptr(a.a_src);
    const char* sbase = uniform_ptr(reinterpret_cast<const char*>(a.ascale));
    const char* wbase;  // weights of the group whose slices `issue` sends
    uint32_t src[C::IPW];
    auto issue = [&](int st, int kt) {
#pragma unroll
        for (int q = 0; q < C::IPW_AB; ++q)
            dma16(__builtin_amdgcn_readfirstlane(lds_base + st * C::STAGE + (q * C::NW + wave) * 1024),
                  op_is_a(q) ? abase : wbase, src[q] + (uint32_t)kt * (op_is_a(q) ? 128u : (uint32_t)C::BROWB));
        if constexpr (C::A8)
            dma4(__builtin_amdgcn_readfirstlane(lds_base + st * C::STAGE + C::A_BYTES + C::B_BYTES + wave * 256),
                 sbase, src[C::IPW_AB] + (uint32_t)kt * 4u);
    };
    // this wave's transfers of a slice have landed while `later` newer slices'
    // transfers (IPW each) may still be in flight
    auto wait_stage = [&](int later) { wait_vmcnt_le<(C::S - 2) * C::IPW>(later * C::IPW); };

    TileInfo cur = decode_tile<C>(a, tile, s_off, s_tile0, G, ntiles_n);
    {
        int idx[C::IPW];
#pragma unroll
        for (int q = 0; q < C::IPW; ++q) idx[q] = a_raw(cur, q);
#pragma unroll
        for (int q = 0; q < C::IPW; ++q) src[q] = source(cur, q, idx[q]);
        wbase = group_weights(cur);
    }
    int ring = 0;  // ring slot of the current tile's slice 0
#pragma unroll
    for (int st = 0; st < C::S - 1; ++st)
        if (st < nk) issue(st, st);

    while (true) {
        const int next_tile = tile + nb;
        const bool has_next = next_tile < total;
        TileInfo nxt = cur;
        int nidx[C::IPW];
        if (has_next) {
            nxt = decode_tile<C>(a, next_tile, s_off, s_tile0, G, ntiles_n);
#pragma unroll
            for (int q = 0; q < C::IPW; ++q) nidx[q] = a_raw(nxt, q);
        }

        f32x4_t acc[C::MI][C::NI];
        f32x4_t part[C::WNARROW ? C::MI : 1][C::WNARROW ? C::NI : 1];  // fp8: this K block's sums
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

        for (int kt = 0; kt < nk; ++kt) {
            wait_stage(min(C::S - 2, nk - 1 - kt));
            lds_barrier();  // slice kt is in LDS for every wave; slot of slice kt-1 is free
            if (kt + C::S - 1 < nk) issue((ring + kt + C::S - 1) % C::S, kt + C::S - 1);
            const char* la = lds + ((ring + kt) % C::S) * C::STAGE;
            const char* lb = la + C::A_BYTES;
            if constexpr (C::A8) {
                // one 128-wide K block: acc += (row scale x weight-block scale) * A.B
                const int sk = a.K / 128;
                const __attribute__((address_space(4))) float* wsp =
                    (const __attribute__((address_space(4))) float*)a.wscale;
                float sw0, sw1;  // weight-block scales of this wave's columns (FC1: gate, up)
                if (MODE == FC1) {
                    const int col = cur.nt * (C::BN / 2);  // the tile's 128 h columns
                    sw0 = wsp[((size_t)cur.g * (a.N / 128) + col / 128) * sk + kt];
                    sw1 = wsp[((size_t)cur.g * (a.N / 128) + (a.I + col) / 128) * sk + kt];
                } else {
                    const int wrow = min(cur.nt * C::BN + wn * C::WTN, a.N - 1);
                    sw0 = sw1 = wsp[((size_t)cur.g * (a.N / 128) + wrow / 128) * sk + kt];
                }
                const float* lsa = reinterpret_cast<const float*>(lb + C::B_BYTES + wave * 256);
                const int g4 = lane >> 4;
                // the result rows of lane l are activation row l % 16 of each
                // 16-row block (operands swapped, see mfma_frag): one row scale
                // per lane and block, times the gate / up (FC1) or the single
                // (FC2) weight-block scale of the wave's columns
                float s0[C::MI], s1[C::MI];
                i32x8_t fa[C::MI];
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi) {
                    const float sa = lsa[mi * 16 + (lane & 15)];
                    s0[mi] = sa * sw0;
                    s1[mi] = sa * sw1;
                    fa[mi] = lds_row32(la, wm * C::WTM + mi * 16 + (lane & 15), g4);
                }
                // Software pipeline: the VALU that scales MFMA result j runs
                // after MFMA j+1 has been issued, so it does not wait for j.
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
                        acc[mi][ni] += ((MODE == FC1 && (ni & 1)) ? s1[mi] : s0[mi]) * pr[jj % (LAGB + 1)];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
                const int kc = ks * 4 + (lane >> 4);
                u32x4_t fa[C::MI], fb[C::NI];
#pragma unroll
                for (int mi = 0; mi < C::MI; ++mi)
                    fa[mi] = *reinterpret_cast<const u32x4_t*>(la + dma_off(wm * C::WTM + mi * 16 + (lane & 15), kc));
#pragma unroll
                for (int ni = 0; ni < C::NI; ++ni) {
                    const int row = wn * C::WTN + ni * 16 + (lane & 15);
                    if constexpr (C::WNARROW) {
                        // 8 fp8 values at K = 32*ks + 8*(lane/16): byte 8*(4*ks + lane/16)
                        // of the 64-byte row, in 16-byte chunk 2*ks + lane/32
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
                if (kt & 1) {
                    // end of a 128-wide K block: acc += block scale * partial.  The
                    // scale index is wave-uniform; the constant address space makes
                    // the loads scalar, so they do not count against the
                    // transfers' vmcnt.
                    const int kb = kt >> 1, sk = a.K / 128;
                    const __attribute__((address_space(4))) float* ws =
                        (const __attribute__((address_space(4))) float*)a.wscale;
#pragma unroll
                    for (int ni = 0; ni < C::NI; ++ni) {
                        const int j = wn * C::WTN + ni * 16;  // first weight row of this block
                        int wrow;
                        if (MODE == FC1) {
                            const int blk = j >> 4, pair = blk >> 1;
                            const int col = cur.nt * (C::BN / 2) + pair * 16;
                            wrow = (blk & 1) ? a.I + col : col;
                        } else {
                            wrow = min(cur.nt * C::BN + j, a.N - 1);
                        }
                        const float sc = ws[((size_t)cur.g * (a.N / 128) + wrow / 128) * sk + kb];
#pragma unroll
                        for (int mi = 0; mi < C::MI; ++mi) {
                            acc[mi][ni] += sc * part[mi][ni];
                            part[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        }
                    }
                }
            }
        }

        // the next tile's first slices go out before this tile's epilogue
        lds_barrier();  // every wave is done reading the ring
        if (has_next) {
#pragma unroll
            for (int q = 0; q < C::IPW; ++q) src[q] = source(nxt, q, nidx[q]);
            wbase = group_weights(nxt);
            ring = (ring + nk) % C::S;
#pragma unroll
            for (int st = 0; st < C::S - 1; ++st)
                if (st < nk) issue((ring + st) % C::S, st);
        }

        // Epilogue.  With the weight fragment as the MFMA's first operand, a
        // 16x16 result block leaves lane l the activation row l%16 and the four
        // consecutive output columns 4*(l/16) + i (i < 4): one 8-byte bf16 write
        // (or a 4-byte fp8 one) per lane and block, no data exchange.
        bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
        const int erow = lane & 15;        // row within a 16x16 block
        const int ecol = (lane >> 4) * 4;  // first of its 4 columns
        if (MODE == FC1 && C::A8) {
            // h -> e4m3 per row and 128 intermediate channels: the tile's 128 h
            // columns are split over the WN wave columns, 4 lanes per row each
            // (lanes l, l^16, l^32, l^48).  h overwrites the gate accumulators.
            float rmax[C::MI];
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi) {
                rmax[mi] = 0.0f;
#pragma unroll
                for (int q = 0; q < C::NI / 2; ++q) {
                    float hv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gt = acc[mi][2 * q][i];
                        const float up = acc[mi][2 * q + 1][i];
                        hv[i] = gt * __builtin_amdgcn_rcpf(1.0f + expf(-gt)) * up;
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[mi][2 * q][i] = hv[i];
                        rmax[mi] = fmaxf(rmax[mi], fabsf(hv[i]));
                    }
                }
                rmax[mi] = fmaxf(rmax[mi], __shfl_xor(rmax[mi], 16, 64));
                rmax[mi] = fmaxf(rmax[mi], __shfl_xor(rmax[mi], 32, 64));
                if (lane < 16) s_amax[(wm * C::WTM + mi * 16 + erow) * C::WN + wn] = rmax[mi];
            }
            lds_barrier();
            uint8_t* hq = reinterpret_cast<uint8_t*>(a.out);
            const int sk_out = a.I / 128;
#pragma unroll
            for (int mi = 0; mi < C::MI; ++mi) {
                float amax = 0.0f;
#pragma unroll
                for (int w = 0; w < C::WN; ++w) amax = fmaxf(amax, s_amax[(wm * C::WTM + mi * 16 + erow) * C::WN + w]);
                const float sc = amax / 448.0f;
                const int rr = cur.m0 + wm * C::WTM + mi * 16 + erow;
                if (rr < cur.nrows) {
                    const size_t r = (size_t)(cur.row0 + rr);
#pragma unroll
                    for (int q = 0; q < C::NI / 2; ++q) {
                        const float hv[4] = {acc[mi][2 * q][0], acc[mi][2 * q][1], acc[mi][2 * q][2], acc[mi][2 * q][3]};
                        const int col = cur.nt * (C::BN / 2) + ((wn * C::WTN) / 32 + q) * 16 + ecol;
                        *(__attribute__((address_space(1))) uint32_t*)(hq + r * a.I + col) = fp8x4_code(hv, sc);
                    }
                    if (wn == 0 && lane < 16) a.out_scale[r * sk_out + cur.nt] = sc;
                }
            }
        } else if (MODE == FC1) {
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
                    const int pair = (wn * C::WTN) / 32 + q;
                    const int col = cur.nt * (C::BN / 2) + pair * 16 + ecol;
                    const int rr = cur.m0 + wm * C::WTM + mi * 16 + erow;
                    if (rr < cur.nrows) store4_bf16(out + (size_t)(cur.row0 + rr) * a.out_ld + col, hv);
                }
        } else {
            // FC2: each wave stages its output 16 rows at a time (bf16) in its
            // share of the ring slot that the next tile fills last, then writes
            // whole 16-byte column chunks, 2*WTN contiguous bytes per row, instead
            // of 8-byte pieces scattered over 16 rows per store instruction.  The
            // region is private to the wave, whose LDS accesses run in order.
            // Non-temporal stores: fc2_out is read back once, by the finalize.
            constexpr int PITCH = C::WTN * 2 + 16;  // staged row bytes (+16 spreads the banks)
            constexpr int CPR = C::WTN / 8;         // 16-byte chunks per row
            constexpr int RPI = 64 / CPR;           // rows per read / store instruction
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
                    const int rr = cur.m0 + wm * C::WTM + mi * 16 + r;
                    // N is a multiple of 16: a 16-byte chunk is wholly inside or outside
                    const int col = cur.nt * C::BN + wn * C::WTN + c * 8;
                    if (rr < cur.nrows && col < a.N)
                        __builtin_nontemporal_store(d, (__attribute__((address_space(1))) u32x4_t*)(out + (size_t)(cur.row0 + rr) * a.out_ld + col));
                }
            }
        }
        // drain: stores and the next tile's first slices; afterwards the stage
        // waits count this block's DMA transfers only
        wait_vmcnt<0>();
        if (!has_next) break;
        tile = next_tile;
        cur = nxt;
    }
}

template <int MODE, class C>
moe_status run_dma_gemm(FfnArgs args, int lo_rows, int hi_rows, int R, hipStream_t s, int kid,
                        int give_max = 0, int take_lo = 0, int take_hi = 0, int take_bm = 0,
                        int take_max = 0)
{
    auto kern = dma_gemm_kernel<MODE, C>;
    static const int occ = [] {  // once per kernel (thread-safe static initialisation)
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dma_gemm_kernel<MODE, C>, C::NT, 0) != hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    args.lo_rows = lo_rows;
    args.hi_rows = hi_rows;
    args.give_max = give_max;
    args.take_lo = take_lo;
    args.take_hi = take_hi;
    args.take_bm = take_bm;
    args.take_max = take_max;
    const long max_tiles = (long)(R / C::BM + args.G) * ((args.N + C::BN - 1) / C::BN);
    long grid = (long)device_cu_count() * occ;
    if (grid > max_tiles) grid = max_tiles;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    {
        TimedLaunch tl(kid, s);
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), 0, s, args);
    }
    return launch_status(MODE == FC1 ? "fc1 dma_gemm_kernel" : "fc2 dma_gemm_kernel");
}

template <class AT, class WT, int MODE, class C>
moe_status run_gemm(FfnArgs args, int lo_rows, int hi_rows, int R, hipStream_t s, int kid)
{
    auto kern = grouped_gemm_kernel<AT, WT, MODE, C>;
    static const int occ = [] {  // once per kernel (thread-safe static initialisation)
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grouped_gemm_kernel<AT, WT, MODE, C>, C::NT, 0) != hipSuccess || n < 1)
            n = 1;
        return n;
    }();
    args.lo_rows = lo_rows;
    args.hi_rows = hi_rows;
    const long max_tiles = (long)(R / C::BM + args.G) * ((args.N + C::BN - 1) / C::BN);
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

// Row classes: each group goes to the tile shape that suits its row count
// (bf16 shapes; the fp8-weight and fp8 x fp8 shapes are listed at their
// dispatch functions below).
//   [0, 64)     32x128 tiles, 4 waves: weight streaming for decode-like groups
//   [64, 384)   128x256 tiles, 16 waves
//   [384, inf)  256x256 tiles, 16 waves: MFMA-bound groups
constexpr int kMidRows = 64;
constexpr int kBigRows = 384;
constexpr int kAllRows = 1 << 30;
constexpr int kHandoffMinK = 4096;  // remainder hand-off between classes from this K on

// bf16 activations with bf16 or fp8 weights: every row class on the
// direct-to-LDS engine.
//
// A big group's last, partial tile goes to the mid launch when it is at most
// 128 rows (and the big tiles are 256 rows high): a mostly-padding 256-row
// tile becomes a 128-row one with half the MFMA work (the weight tile is
// read once either way).  The same hand-off from mid to skinny tiles was
// measured and is not used: a 32-row tile streams the weights again with a
// quarter of the waves (fp8 x fp8 Qwen3-shaped FC1 +13%).
template <int MODE, class Skinny, class Mid, class Big>
moe_status run_classes_dma(const FfnArgs& f, int R, hipStream_t s, int kid)
{
    static_assert(Skinny::BM < Mid::BM && Mid::BM <= Big::BM, "tile heights grow with the class");
    // Only for long K: a tile's fixed costs (ring fill, epilogue) are then small
    // against its MFMA work, so a shorter tile pays.  Measured: FC2 of the
    // Mixtral-shaped layer (K = 14336) -10%, FC1 of the fp8 x fp8 DeepSeek-V3
    // prefill (K = 7168) -2.5%; with K = 2048 (DeepSeek-V3 FC2) +2.5%.
    const bool handoff = f.K >= kHandoffMinK;
    const int big_give = (handoff && Big::BM > Mid::BM) ? Mid::BM : 0;  // none when the shapes match
    moe_status st = run_dma_gemm<MODE, Skinny>(f, 0, kMidRows, R, s, kid);
    if (st != MOE_OK) return st;
    st = run_dma_gemm<MODE, Mid>(f, kMidRows, kBigRows, R, s, kid, 0, kBigRows, kAllRows, Big::BM,
                                 big_give);
    if (st != MOE_OK) return st;
    return run_dma_gemm<MODE, Big>(f, kBigRows, kAllRows, R, s, kid, big_give);
}

// Shapes chosen by measurement on MI355X: 4 waves per SIMD for the large tiles
// (one wave alone cannot keep the MFMA pipe busy), whole-line requests, and for
// the weight-streaming skinny tiles a narrow 32x128 tile with a 6-deep ring
// (5 slices, 100 KB, in flight per CU).
template <int MODE>
moe_status run_classes_bf16(const FfnArgs& f, int R, hipStream_t s, int kid)
{
    return run_classes_dma<MODE, DmaCfg<32, 128, 1, 4, 2, 6>, DmaCfg<128, 256, 4, 4, 2, 3>,
                           DmaCfg<256, 256, 4, 4, 4, 2>>(f, R, s, kid);
}

// fp8 weights keep a second (per-scale-block) accumulator set, which does not
// fit a 256x256 tile's registers: big groups use the 128x256 shape too, with
// 8 waves of 64x64 (fewer LDS bytes per MFMA than 16 waves of 32x64: -4%
// time measured).  Half as many weight bytes per stage allow deeper rings.
template <int MODE>
moe_status run_classes_w8(const FfnArgs& f, int R, hipStream_t s, int kid)
{
    return run_classes_dma<MODE, DmaCfg<32, 256, 1, 4, 2, 6, true>, DmaCfg<128, 256, 2, 4, 2, 4, true>,
                           DmaCfg<128, 256, 2, 4, 4, 4, true>>(f, R, s, kid);
}

template <class AT, class WT>
moe_status run_ffn(const FfnArgs& fc1, const FfnArgs& fc2, int R, hipStream_t s);

template <>
moe_status run_ffn<bf16_t, bf16_t>(const FfnArgs& fc1, const FfnArgs& fc2, int R, hipStream_t s)
{
    moe_status st = run_classes_bf16<FC1>(fc1, R, s, MOE_KID_FC1);
    if (st != MOE_OK) return st;
    return run_classes_bf16<FC2>(fc2, R, s, MOE_KID_FC2);
}

template <>
moe_status run_ffn<bf16_t, fp8_t>(const FfnArgs& fc1, const FfnArgs& fc2, int R, hipStream_t s)
{
    moe_status st = run_classes_w8<FC1>(fc1, R, s, MOE_KID_FC1);
    if (st != MOE_OK) return st;
    return run_classes_w8<FC2>(fc2, R, s, MOE_KID_FC2);
}

// fp8 activations and weights: every class on fp8 MFMA, 256-column tiles (one
// 128-channel block of h per FC1 tile).  Big groups: 8 waves of 64x128
// (16 waves of 64x64 would not fit their operands and accumulators in 128
// VGPRs); mid: 8 waves of 64x64; skinny: 32x256 with a 4-deep ring.
template <int MODE>
moe_status run_classes_a8(const FfnArgs& f, int R, hipStream_t s, int kid)
{
    return run_classes_dma<MODE, DmaCfg<32, 256, 1, 4, 2, 4, true, true>, DmaCfg<128, 256, 2, 4, 2, 3, true, true>,
                           DmaCfg<256, 256, 4, 2, 4, 2, true, true>>(f, R, s, kid);
}

// fp32 (small reference-precision layers): one 32x128 tile shape for all groups.
template <>
moe_status run_ffn<float, float>(const FfnArgs& fc1, const FfnArgs& fc2, int R, hipStream_t s)
{
    using C = Cfg<float, float, 32, 128, 1, 4, 1>;
    moe_status st = run_gemm<float, float, FC1, C>(fc1, 0, kAllRows, R, s, MOE_KID_FC1);
    if (st != MOE_OK) return st;
    return run_gemm<float, float, FC2, C>(fc2, 0, kAllRows, R, s, MOE_KID_FC2);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

size_t ffn_fp8_scratch_bytes(int T, int k, int n_shared, int I)
{
    const size_t R = (size_t)T * k + (size_t)n_shared * T;
    return align256(R * (size_t)I) + align256(R * (size_t)(I / 128) * 4);
}

moe_status launch_ffn_fp8(const uint8_t* xq, const float* x_scale, int T, int H, int I, int k, int E,
                          int n_shared, const int32_t* offsets, const int32_t* permuted_pair,
                          const uint8_t* w13, const uint8_t* w2, const float* w13_scale,
                          const float* w2_scale, void* fc2_out, void* ws, hipStream_t s)
{
    const int G = E + n_shared;
    const int R = T * k + n_shared * T;
    char* hq = static_cast<char*>(ws);
    float* hs = reinterpret_cast<float*>(hq + align256((size_t)R * I));
    FfnArgs f1{};
    f1.a_src = reinterpret_cast<const char*>(xq);
    f1.ascale = x_scale;
    f1.w = reinterpret_cast<const char*>(w13);
    f1.wscale = w13_scale;
    f1.out = hq;
    f1.out_scale = hs;
    f1.offsets = offsets;
    f1.permuted_pair = permuted_pair;
    f1.T = T; f1.k = k; f1.E = E; f1.G = G; f1.I = I;
    f1.N = 2 * I; f1.K = H; f1.out_ld = I;
    FfnArgs f2 = f1;
    f2.a_src = hq;
    f2.ascale = hs;
    f2.w = reinterpret_cast<const char*>(w2);
    f2.wscale = w2_scale;
    f2.out = static_cast<char*>(fc2_out);
    f2.out_scale = nullptr;
    f2.N = H; f2.K = I; f2.out_ld = H;
    moe_status st = run_classes_a8<FC1>(f1, R, s, MOE_KID_FC1);
    if (st != MOE_OK) return st;
    return run_classes_a8<FC2>(f2, R, s, MOE_KID_FC2);
}

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
    if (act == MOE_F32) return run_ffn<float, float>(f1, f2, R, s);
    if (wdt == MOE_FP8_E4M3) return run_ffn<bf16_t, fp8_t>(f1, f2, R, s);
    return run_ffn<bf16_t, bf16_t>(f1, f2, R, s);
}

}  // namespace moe
